"""Seeded synthetic decode workloads (inputs only; none of the attention
arithmetic lives here).

Five workloads, each a decode batch (one query token per sequence) over a
paged KV cache in the layouts of the page "BI-V100 PagedAttention V2
implementation" (key_cache [num_blocks, Hkv, D/x, bs, x], value_cache
[num_blocks, Hkv, D, bs]):

  1 tiny_fp32        B=2,   H=4,  Hkv=2,  D=64,  bs=16, fp32, L={37, 700},
                     a 64-block pool assigned by a seeded permutation
  2 gqa_bf16         B=64,  H=28, Hkv=4,  D=128, bs=16, bf16, L ~ U[1024, 8192]
  3 long_fp16        B=4,   H=32, Hkv=8,  D=128, bs=16, fp16, L = 100000,
                     values 0.5 * N(0, 1)
  4 ragged_alibi_bf16 B=256, H=Hkv=32,   D=128, bs=16, bf16,
                     L = clip(round(lognormal(ln 2048, 1.0)), 16, 32768),
                     ALiBi slopes 2^(-8 (h+1) / 32)
  5 fp8_kv           B=32,  H=64, Hkv=8,  D=128, bs=32, bf16 query/out,
                     OCP FP8 E4M3FN cache quantised per tensor with
                     scale = amax / 448 (round to nearest even, saturating),
                     L = 32768

Recipe: sequence lengths and the block pool's permutation come from NumPy's
PCG64 seeded with 1000 + k (k = workload number); query / key / value values
come from a torch generator on the target device seeded the same way, drawn
as float32 N(0, 1) (times the workload's std) and rounded to the storage
type.  Pools hold exactly sum(ceil(L / bs)) blocks (workload 1: 64),
shuffled; blocks are assigned to sequences in order.  Unused block-table
entries are 0, or point at an all-NaN sentinel block when ``poison`` is set
(then the pool's unused blocks and the slots past each sequence's end are
NaN as well).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

PARTITION_SIZE = 512
FP8_MAX = 448.0

WORKLOADS = {
    1: dict(name="tiny_fp32", B=2, H=4, Hkv=2, D=64, bs=16, dtype=torch.float32, kv="auto",
            std=1.0, lens="fixed", fixed=(37, 700), pool=64, alibi=False),
    2: dict(name="gqa_bf16", B=64, H=28, Hkv=4, D=128, bs=16, dtype=torch.bfloat16, kv="auto",
            std=1.0, lens="uniform", lo=1024, hi=8192, alibi=False),
    3: dict(name="long_fp16", B=4, H=32, Hkv=8, D=128, bs=16, dtype=torch.float16, kv="auto",
            std=0.5, lens="fixed", fixed=(100000,) * 4, alibi=False),
    4: dict(name="ragged_alibi_bf16", B=256, H=32, Hkv=32, D=128, bs=16, dtype=torch.bfloat16,
            kv="auto", std=1.0, lens="lognormal", median=2048, sigma=1.0, lo=16, hi=32768,
            alibi=True),
    5: dict(name="fp8_kv", B=32, H=64, Hkv=8, D=128, bs=32, dtype=torch.bfloat16, kv="fp8_e4m3",
            std=1.0, lens="fixed", fixed=(32768,) * 32, alibi=False),
}

STORAGE_KIND = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


@dataclass
class Workload:
    number: int
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    dtype: torch.dtype
    kv_cache_dtype: str                 # "auto" or "fp8_e4m3"
    query: torch.Tensor                 # [B, H, D] dtype
    key_cache: torch.Tensor             # [NB, Hkv, D/x, bs, x] (uint8 for fp8)
    value_cache: torch.Tensor           # [NB, Hkv, D, bs]
    block_tables: torch.Tensor          # int32 [B, max_blocks]
    seq_lens: torch.Tensor              # int32 [B]
    lens: np.ndarray                    # host copy of seq_lens
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    alibi_slopes: Optional[torch.Tensor] = None
    max_seq_len: int = 0
    max_num_partitions: int = 1
    poison_block: Optional[int] = None
    extras: dict = field(default_factory=dict)

    @property
    def kv_elem_bytes(self) -> int:
        return 1 if self.kv_cache_dtype == "fp8_e4m3" else torch.tensor([], dtype=self.dtype).element_size()

    @property
    def kv_kind(self) -> str:
        return "fp8_e4m3" if self.kv_cache_dtype == "fp8_e4m3" else STORAGE_KIND[self.dtype]

    @property
    def q_kind(self) -> str:
        return STORAGE_KIND[self.dtype]

    def kv_bytes(self) -> int:
        """Bytes of K and V the live tokens occupy (each read once per KV head)."""
        return int(self.lens.sum()) * self.num_kv_heads * self.head_size * 2 * self.kv_elem_bytes

    def alloc_outputs(self, partials: str = "f32"):
        """out, exp_sums, max_logits, tmp_out on the workload's device; tmp_out
        is float32 (``partials="f32"``, the default) or in the query dtype
        (``"out"``)."""
        dev = self.query.device
        b, h, d, p = self.num_seqs, self.num_heads, self.head_size, self.max_num_partitions
        out = torch.empty((b, h, d), dtype=self.dtype, device=dev)
        exp_sums = torch.empty((b, h, p), dtype=torch.float32, device=dev)
        max_logits = torch.empty((b, h, p), dtype=torch.float32, device=dev)
        if partials not in ("f32", "out"):
            raise ValueError("partials must be 'f32' or 'out'")
        tdt = torch.float32 if partials == "f32" else self.dtype
        tmp_out = torch.empty((b, h, p, d), dtype=tdt, device=dev)
        return out, exp_sums, max_logits, tmp_out


def draw_lengths(spec: dict, rng: np.random.Generator, num_seqs: int) -> np.ndarray:
    kind = spec["lens"]
    if kind == "fixed":
        base = np.array(spec["fixed"], dtype=np.int64)
        return np.resize(base, num_seqs)
    if kind == "uniform":
        return rng.integers(spec["lo"], spec["hi"] + 1, size=num_seqs).astype(np.int64)
    if kind == "lognormal":
        raw = rng.lognormal(mean=math.log(spec["median"]), sigma=spec["sigma"], size=num_seqs)
        return np.clip(np.round(raw), spec["lo"], spec["hi"]).astype(np.int64)
    raise ValueError(kind)


def _fill_random(dst: torch.Tensor, gen: torch.Generator, std: float, chunk_rows: int = 2048):
    """dst[:] = round_to_dtype(std * N(0,1)), generated row-chunk by row-chunk."""
    for r0 in range(0, dst.shape[0], chunk_rows):
        r1 = min(dst.shape[0], r0 + chunk_rows)
        shape = (r1 - r0,) + tuple(dst.shape[1:])
        vals = torch.randn(shape, generator=gen, dtype=torch.float32, device=dst.device)
        if std != 1.0:
            vals.mul_(std)
        dst[r0:r1].copy_(vals)


def _fill_fp8(dst_u8: torch.Tensor, gen: torch.Generator, std: float, chunk_rows: int = 1024):
    """Quantise std * N(0,1) to E4M3FN with one per-tensor scale amax / 448.

    Two passes over the same generator state: the first finds amax, the
    second quantises (round to nearest even via torch's float8 cast, after
    clamping to the finite range).  Returns the scale."""
    state = gen.get_state()
    amax = 0.0
    for r0 in range(0, dst_u8.shape[0], chunk_rows):
        r1 = min(dst_u8.shape[0], r0 + chunk_rows)
        vals = torch.randn((r1 - r0,) + tuple(dst_u8.shape[1:]), generator=gen,
                           dtype=torch.float32, device=dst_u8.device) * std
        amax = max(amax, float(vals.abs().max()))
    scale = amax / FP8_MAX
    gen.set_state(state)
    for r0 in range(0, dst_u8.shape[0], chunk_rows):
        r1 = min(dst_u8.shape[0], r0 + chunk_rows)
        vals = torch.randn((r1 - r0,) + tuple(dst_u8.shape[1:]), generator=gen,
                           dtype=torch.float32, device=dst_u8.device) * std
        q = (vals / scale).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
        dst_u8[r0:r1].copy_(q.view(torch.uint8))
    return scale


def make_workload(number: int, device="cuda", *, num_seqs: Optional[int] = None,
                  lens: Optional[list] = None, poison: bool = False,
                  seed: Optional[int] = None, **overrides) -> Workload:
    """Builds workload ``number`` (1..5) on ``device``.

    ``num_seqs`` / ``lens`` shrink or override the batch (the other recipe
    choices stay); ``overrides`` replace recipe entries (H, Hkv, D, bs, dtype,
    kv, std, alibi); ``poison`` adds an all-NaN sentinel block that every
    unused block-table entry points at, and NaN-fills unused pool blocks and
    the tail slots past each sequence's end.
    """
    spec = dict(WORKLOADS[number])
    unknown = set(overrides) - set(spec)
    if unknown:
        raise ValueError(f"unknown workload overrides {sorted(unknown)}")
    spec.update(overrides)
    seed = 1000 + number if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    b = spec["B"] if num_seqs is None else num_seqs
    seq_lens = np.asarray(lens, dtype=np.int64) if lens is not None else draw_lengths(spec, rng, b)
    b = len(seq_lens)
    hkv, h, d, bs = spec["Hkv"], spec["H"], spec["D"], spec["bs"]
    need = (seq_lens + bs - 1) // bs
    used = int(need.sum())
    pool = max(used, 1)
    if lens is None and num_seqs is None and "pool" in spec:
        pool = max(pool, spec["pool"])
    perm = rng.permutation(pool)
    sentinel = pool if poison else None
    total_blocks = pool + (1 if poison else 0)
    max_seq_len = int(seq_lens.max(initial=0))
    max_blocks = max(1, (max_seq_len + bs - 1) // bs)
    tables = np.full((b, max_blocks), sentinel if poison else 0, dtype=np.int32)
    off = 0
    for s in range(b):
        tables[s, :need[s]] = perm[off:off + need[s]]
        off += need[s]

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dtype = spec["dtype"]
    fp8 = spec["kv"] == "fp8_e4m3"
    elem = 1 if fp8 else torch.tensor([], dtype=dtype).element_size()
    x = 16 // elem
    query = torch.empty((b, h, d), dtype=dtype, device=device)
    _fill_random(query, gen, spec["std"])
    kshape = (total_blocks, hkv, d // x, bs, x)
    vshape = (total_blocks, hkv, d, bs)
    k_scale = v_scale = 1.0
    if fp8:
        key_cache = torch.empty(kshape, dtype=torch.uint8, device=device)
        value_cache = torch.empty(vshape, dtype=torch.uint8, device=device)
        k_scale = _fill_fp8(key_cache[:pool], gen, spec["std"])
        v_scale = _fill_fp8(value_cache[:pool], gen, spec["std"])
    else:
        key_cache = torch.empty(kshape, dtype=dtype, device=device)
        value_cache = torch.empty(vshape, dtype=dtype, device=device)
        _fill_random(key_cache[:pool], gen, spec["std"])
        _fill_random(value_cache[:pool], gen, spec["std"])
    if poison:
        _poison(key_cache, value_cache, tables, seq_lens, bs, pool, fp8)

    alibi = None
    if spec["alibi"]:
        alibi = torch.tensor([2.0 ** (-8.0 * (i + 1) / h) for i in range(h)], dtype=torch.float32,
                             device=device)
    wl = Workload(
        number=number, name=spec["name"], num_seqs=b, num_heads=h, num_kv_heads=hkv,
        head_size=d, block_size=bs, dtype=dtype, kv_cache_dtype=spec["kv"], query=query,
        key_cache=key_cache, value_cache=value_cache,
        block_tables=torch.from_numpy(tables).to(device),
        seq_lens=torch.from_numpy(seq_lens.astype(np.int32)).to(device), lens=seq_lens,
        scale=1.0 / math.sqrt(d), k_scale=k_scale, v_scale=v_scale, alibi_slopes=alibi,
        max_seq_len=max_seq_len,
        max_num_partitions=max(1, (max_seq_len + PARTITION_SIZE - 1) // PARTITION_SIZE),
        poison_block=sentinel)
    return wl


def _poison(key_cache, value_cache, tables, seq_lens, bs, pool, fp8):
    """NaN into the sentinel block, the unused pool blocks and the tail slots."""
    nan_k = 0x7F if fp8 else float("nan")
    used = set()
    for s in range(tables.shape[0]):
        n = (int(seq_lens[s]) + bs - 1) // bs
        used.update(int(v) for v in tables[s, :n])
    unused = [i for i in range(pool) if i not in used] + [pool]
    idx = torch.tensor(unused, dtype=torch.long, device=key_cache.device)
    key_cache.index_fill_(0, idx, nan_k)
    value_cache.index_fill_(0, idx, nan_k)
    for s in range(tables.shape[0]):
        L = int(seq_lens[s])
        if L % bs:
            last = int(tables[s, (L + bs - 1) // bs - 1])
            key_cache[last, :, :, L % bs:, :] = nan_k
            value_cache[last, :, :, L % bs:] = nan_k


def to_block_rows(key_cache: torch.Tensor, value_cache: torch.Tensor):
    """The same 16-bit caches repacked from the decode layout (K [NB, Hkv, D/x,
    bs, x], V [NB, Hkv, D, bs]) into the [NB, Hkv, bs, D] block-rows layout
    (a copy; values unchanged)."""
    nb, hkv, dx, bs, x = key_cache.shape
    k = key_cache.permute(0, 1, 3, 2, 4).reshape(nb, hkv, bs, dx * x).contiguous()
    v = value_cache.permute(0, 1, 3, 2).contiguous()
    return k, v


def raw_storage(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's storage words as the oracle reads them."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def host_subset(wl: Workload, seqs) -> dict:
    """Raw host storage of the listed sequences only, with a compacted pool.

    Returns dict(query, key_cache, value_cache, block_tables, seq_lens) where
    the block tables index the compacted pool (rows of other sequences are
    empty).  Used to hand large workloads to the CPU oracle a few sequences at
    a time; the bytes are exactly those the GPU reads.
    """
    bs = wl.block_size
    tables = wl.block_tables.cpu().numpy()
    blocks, new_tables = [], np.zeros_like(tables)
    for s in seqs:
        n = (int(wl.lens[s]) + bs - 1) // bs
        new_tables[s, :n] = np.arange(len(blocks), len(blocks) + n)
        blocks.extend(int(v) for v in tables[s, :n])
    idx = torch.tensor(blocks if blocks else [0], dtype=torch.long, device=wl.key_cache.device)
    return dict(query=raw_storage(wl.query), key_cache=raw_storage(wl.key_cache[idx]),
                value_cache=raw_storage(wl.value_cache[idx]), block_tables=new_tables,
                seq_lens=wl.lens.copy())


# --------------------------------------------------------------------------
# Prefill batches (inputs only)
# --------------------------------------------------------------------------

#: Prefill workloads: query / key counts per sequence and the model shape.
#:   prefill_bf16   8 prompts of 2048 tokens (nq = nk = 2048), H=32, Hkv=8,
#:                  D=128, bs=16, bf16, causal: a fresh prefill
#:   chunked_bf16   16 sequences, 512 new tokens over 8192-token contexts
#:                  (nq = 512, nk = 8192), same model shape: chunked prefill
PREFILL_WORKLOADS = {
    "prefill_bf16": dict(qlens=(2048,) * 8, klens=(2048,) * 8, H=32, Hkv=8, D=128, bs=16,
                         dtype=torch.bfloat16),
    "chunked_bf16": dict(qlens=(512,) * 16, klens=(8192,) * 16, H=32, Hkv=8, D=128, bs=16,
                         dtype=torch.bfloat16),
}


@dataclass
class PrefillWorkload:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    dtype: torch.dtype
    query: torch.Tensor          # [total_q, H, D]
    key_cache: torch.Tensor      # [NB, Hkv, bs, D]
    value_cache: torch.Tensor    # [NB, Hkv, bs, D]
    block_tables: torch.Tensor   # int32 [B, max_blocks]
    cu_seq_q: torch.Tensor       # int32 [B + 1]
    cu_seq_k: torch.Tensor       # int32 [B + 1]
    qlens: np.ndarray
    klens: np.ndarray
    scale: float

    @property
    def max_seq_q(self) -> int:
        return int(self.qlens.max(initial=0))

    @property
    def max_seq_k(self) -> int:
        return int(self.klens.max(initial=0))

    @property
    def kind(self) -> str:
        return STORAGE_KIND[self.dtype]


def make_prefill_workload(name: str = "prefill_bf16", device="cuda", *, qlens=None, klens=None,
                          seed: int = 2000, **overrides) -> PrefillWorkload:
    """Seeded prefill batch: N(0, 1) query / key / value values rounded to the
    dtype (torch generator on ``device``), a shuffled block pool holding
    exactly the blocks the sequences need (NumPy PCG64)."""
    spec = dict(PREFILL_WORKLOADS[name])
    if qlens is not None:
        spec["qlens"] = tuple(qlens)
    if klens is not None:
        spec["klens"] = tuple(klens)
    spec.update(overrides)
    ql = np.asarray(spec["qlens"], dtype=np.int64)
    kl = np.asarray(spec["klens"], dtype=np.int64)
    b, h, hkv, d, bs, dtype = len(ql), spec["H"], spec["Hkv"], spec["D"], spec["bs"], spec["dtype"]
    rng = np.random.Generator(np.random.PCG64(seed))
    need = (kl + bs - 1) // bs
    pool = max(int(need.sum()), 1)
    perm = rng.permutation(pool)
    tables = np.zeros((b, max(1, int(need.max(initial=0)))), dtype=np.int32)
    off = 0
    for s in range(b):
        tables[s, :need[s]] = perm[off:off + need[s]]
        off += need[s]
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    query = torch.empty((int(ql.sum()), h, d), dtype=dtype, device=device)
    key_cache = torch.empty((pool, hkv, bs, d), dtype=dtype, device=device)
    value_cache = torch.empty((pool, hkv, bs, d), dtype=dtype, device=device)
    for t in (query, key_cache, value_cache):
        _fill_random(t, gen, 1.0)
    cu_q = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(kl)]).astype(np.int32)
    return PrefillWorkload(
        name=name, num_seqs=b, num_heads=h, num_kv_heads=hkv, head_size=d, block_size=bs,
        dtype=dtype, query=query, key_cache=key_cache, value_cache=value_cache,
        block_tables=torch.from_numpy(tables).to(device),
        cu_seq_q=torch.from_numpy(cu_q).to(device), cu_seq_k=torch.from_numpy(cu_k).to(device),
        qlens=ql, klens=kl, scale=1.0 / math.sqrt(d))


def prefill_host_subset(wl: PrefillWorkload, seqs) -> dict:
    """Raw host storage of the listed sequences (queries and a compacted pool)
    for the CPU oracle: dict(query, key_cache, value_cache, block_tables,
    cu_seq_q, cu_seq_k, rows) with ``rows`` the global query rows kept."""
    bs = wl.block_size
    tables = wl.block_tables.cpu().numpy()
    cu_q = np.concatenate([[0], np.cumsum(wl.qlens)])
    blocks, rows = [], []
    new_tables = np.zeros((len(seqs), tables.shape[1]), dtype=np.int32)
    qlens, klens = [], []
    for i, s in enumerate(seqs):
        n = (int(wl.klens[s]) + bs - 1) // bs
        new_tables[i, :n] = np.arange(len(blocks), len(blocks) + n)
        blocks.extend(int(v) for v in tables[s, :n])
        rows.extend(range(int(cu_q[s]), int(cu_q[s + 1])))
        qlens.append(int(wl.qlens[s]))
        klens.append(int(wl.klens[s]))
    idx = torch.tensor(blocks if blocks else [0], dtype=torch.long, device=wl.key_cache.device)
    ridx = torch.tensor(rows if rows else [0], dtype=torch.long, device=wl.query.device)
    return dict(query=raw_storage(wl.query[ridx]), key_cache=raw_storage(wl.key_cache[idx]),
                value_cache=raw_storage(wl.value_cache[idx]), block_tables=new_tables,
                cu_seq_q=np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32),
                cu_seq_k=np.concatenate([[0], np.cumsum(klens)]).astype(np.int32),
                rows=np.asarray(rows, dtype=np.int64))
