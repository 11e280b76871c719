"""The oracle against its pins (CPU only): brute force, closed forms,
library routines, the pages' invariants and worked examples."""

import itertools

import pytest

from tests import oracle_pins as P

LENGTHS = [1, 15, 16, 17, 511, 512, 513, 1100]
KINDS = ["f32", "bf16", "f16", "fp8_e4m3"]
GRID = list(itertools.product([16, 32], [1, 2, 7, 8], [64, 128]))


@pytest.mark.parametrize("bs,group,head_size", GRID)
def test_brute_force_grid(bs, group, head_size):
    """Oracle on paged storage == dense softmax attention, across the length,
    block-size, group and head-size grid; storage kind and ALiBi vary by case."""
    i = GRID.index((bs, group, head_size))
    kind = KINDS[i % len(KINDS)]
    alibi = (i // len(KINDS)) % 2 == 1
    k_scale, v_scale = ((0.5, 2.0) if kind == "fp8_e4m3" else (1.0, 1.0))
    hkv = 1 if group >= 7 else 2
    P.pin_brute_force(LENGTHS, hkv, group, head_size, bs, kind, alibi=alibi,
                      k_scale=k_scale, v_scale=v_scale, seed=100 + i)


@pytest.mark.parametrize("args", P.BRUTE_FORCE_SMALL)
def test_brute_force_small(args):
    P.pin_brute_force(*args)


def test_fp8_special_values():
    P.pin_fp8_special_values()


def test_storage_decode():
    P.pin_storage_decode()


def test_partition_statistics():
    P.pin_partition_statistics()


def test_partition_statistics_no_alibi_bf16():
    P.pin_partition_statistics(lens=(600, 1024, 3), kv_kind="bf16", alibi=False)


def test_uniform_closed_form():
    P.pin_uniform_closed_form()


def test_alibi_closed_form():
    P.pin_alibi_closed_form()


def test_single_token():
    P.pin_single_token()


def test_partition_size_independence():
    P.pin_partition_size_independence()


def test_v2_single_partition_equals_v1():
    P.pin_v2_single_partition_equals_v1()


def test_block_table_permutation():
    P.pin_block_table_permutation()


def test_convexity_and_dominant_key():
    P.pin_convexity_and_dominant_key()


def test_empty_sequence():
    P.pin_empty_sequence()


def test_dispatch_golden():
    P.pin_dispatch_golden()


def test_partition_count_golden():
    P.pin_partition_count_golden()


def test_sliding_window():
    P.pin_sliding_window()


def test_sliding_window_with_soft_cap():
    P.pin_sliding_window(lens=(513, 1100), alibi=False, cap=5.0)


def test_soft_cap_forms():
    P.pin_soft_cap_forms()


def test_window_and_cap_every_kind():
    P.pin_window_and_cap_brute_force()
