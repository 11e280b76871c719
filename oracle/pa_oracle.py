"""Plain fp64 CPU oracle for paged-attention decode (v1 and partitioned v2).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
executes this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code with the HIP library and imports
nothing from it (NumPy only, no torch).

Sources (the pages are cited by title and section; no line numbers):

* "BI-V100 PagedAttention V2 implementation" -- the commit page of
  ``paged_attention_v2_pytorch.py`` (called "the V2 page" below): the module
  docstring ("Algorithm", "Performance vs V1", "Correctness"), the argument
  list of ``paged_attention_v2_pytorch`` (cache layouts, block tables,
  ``kv_cache_dtype``/``k_scale``/``v_scale``), the per-block gather loop,
  the GQA expansion, "Phase 1: Per-partition attention", the padding of unused
  partitions and "Phase 2: Reduce across partitions (log-sum-exp)".
* "ex_engine/factors/attn_dispatch.py" -- "Layer 3: Attention prefill/decode
  dispatch" (called "the dispatch page"): the PyTorch decode fallback of
  ``dispatch_decode`` (gather, GQA expand, softmax(q.K * scale).V), which is a
  plain whole-sequence (v1) definition of the output.

Readings where the pages are silent, ambiguous or contradict themselves
(every one is listed with its reason in the design notes of the repository):

* The partition output O_p is NORMALISED by its own exp-sum S_p.  The printed
  code of the V2 page stores the un-normalised weighted sum and then multiplies
  by S_p again in the merge, which double counts and contradicts the page's
  own text ("compute QK^T, softmax, weighted V sum"; "equivalent to full
  softmax"; "tested against V1").  With a normalised O_p the page's merge
  formula  out = sum_p (exp(m_p - M) S_p / sum_q exp(m_q - M) S_q) O_p  is
  exactly the full softmax.
* The number of partitions is ceil(L / 512) (the page's code); the prose
  figure "195" for L = 100000 is a rounding slip (ceil gives 196).
* ALiBi adds slope_h * t with t the absolute 0-based key position, after the
  scale (V2 page, "Alibi bias" step of Phase 1).
* GQA maps query head h to KV head h // (H / Hkv) (``repeat_interleave``).
* The K cache packs x = 16 / sizeof(element) consecutive head dims in its last
  axis: dim d = c * x + j for index [.., c, t, j].
* Padding partitions p >= P_s hold max_logit = -inf, exp_sum = 0, O = 0.
* seq_len = 0 gives an all-zero output row and padding statistics.
* The KV element decoded from storage is multiplied by k_scale / v_scale
  (V2 page applies them to the gathered keys/values).  fp8 storage is OCP
  E4M3FN (bias 7, no infinities, S.1111.111 is NaN).
* The attention weights are NOT rounded to the V dtype before the weighted
  sum (the page's ``.to(v_part.dtype)``): this oracle is exact fp64; the GPU's
  rounding of P is covered by the stated tolerances.
* Sliding window and logit soft cap (the dispatch page's decode configuration
  fields ``window_left`` / ``softcap``, which the pages pass on but do not
  define; the Neuron page hands the same pair to ``flash_attn_varlen_func`` as
  ``window_size`` / ``softcap``, whose meaning is taken): with window_left
  W >= 0 the decode query (position L - 1) sees the keys t >= L - 1 - W only
  (W = -1: no window; a right window is moot for the last token); with
  soft cap c > 0 each scaled logit s becomes c * tanh(s / c), before the ALiBi
  bias is added.  Partitions with no visible key hold -inf, 0, 0 like the
  padding partitions.

Every function works on NumPy arrays; floating point is float64 throughout.
"""

from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

#: Tokens per partition ("_PARTITION_SIZE = 512", V2 page module constants).
PARTITION_SIZE = 512

#: Storage kinds understood by :func:`decode_storage`.
STORAGE_KINDS = ("f32", "f16", "bf16", "fp8_e4m3")


# --------------------------------------------------------------------------
# Storage decoding
# --------------------------------------------------------------------------

def fp8_e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 OCP FP8 E4M3FN codes, as float64.

    Written from the OCP 8-bit floating point definition (E4M3 variant with
    "FN" encodings): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 encodes subnormals m/8 * 2^-6; exponent field 15 with
    mantissa 7 is NaN; there is no infinity, so S.1111.000..110 are the finite
    values 256..448.  The V2 page only names ``kv_cache_dtype`` and the
    per-tensor ``k_scale``/``v_scale``; the byte format is this reading.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if (code >> 7) & 1 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            table[code] = math.nan
        elif exp_field == 0:
            table[code] = sign * (mant / 8.0) * 2.0 ** (1 - 7)
        else:
            table[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return table


_FP8_TABLE = fp8_e4m3fn_table()


def decode_storage(raw: np.ndarray, kind: str) -> np.ndarray:
    """Decode raw storage words to float64.

    ``raw`` holds the bytes exactly as they sit in device memory:
    float32 values for ``"f32"``; uint16 bit patterns for ``"f16"`` (IEEE
    binary16) and ``"bf16"`` (the upper half of an IEEE binary32); uint8 codes
    for ``"fp8_e4m3"``.
    """
    if kind == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if kind == "f16":
        return np.asarray(raw, dtype=np.uint16).view(np.float16).astype(np.float64)
    if kind == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):
            return bits.view(np.float32).astype(np.float64)
    if kind == "fp8_e4m3":
        return _FP8_TABLE[np.asarray(raw, dtype=np.uint8)]
    raise ValueError(f"unknown storage kind {kind!r}")


# --------------------------------------------------------------------------
# Block gather (V2 page: argument list and the per-block gather loop)
# --------------------------------------------------------------------------

def num_partitions(seq_len: int, partition_size: int = PARTITION_SIZE) -> int:
    """ceil(seq_len / partition_size) (V2 page, Phase 1 partition count)."""
    return (seq_len + partition_size - 1) // partition_size


def gather_sequence(key_cache: np.ndarray, value_cache: np.ndarray,
                    block_table_row: np.ndarray, seq_len: int,
                    block_size: int):
    """Gather one sequence's keys and values through its block table.

    key_cache   [num_blocks, Hkv, D/x, block_size, x]  (already decoded)
    value_cache [num_blocks, Hkv, D, block_size]       (already decoded)
    Token t lives in slot t % block_size of logical block t // block_size,
    whose physical block is block_table_row[t // block_size]; only the first
    ceil(seq_len / block_size) entries are read.

    Returns K, V as float64 arrays of shape [seq_len, Hkv, D].
    """
    num_blocks, hkv, d_over_x, bs, x = key_cache.shape
    assert bs == block_size and value_cache.shape[3] == block_size
    head_size = d_over_x * x
    n_logical = (seq_len + block_size - 1) // block_size
    phys = np.asarray(block_table_row[:n_logical], dtype=np.int64)
    assert np.all((phys >= 0) & (phys < num_blocks)), "block table entry out of range"
    # [n, Hkv, D/x, bs, x] -> [n, bs, Hkv, D/x, x] -> [n*bs, Hkv, D]
    k = key_cache[phys].transpose(0, 3, 1, 2, 4).reshape(n_logical * block_size, hkv, head_size)
    # [n, Hkv, D, bs] -> [n, bs, Hkv, D] -> [n*bs, Hkv, D]
    v = value_cache[phys].transpose(0, 3, 1, 2).reshape(n_logical * block_size, hkv, head_size)
    return k[:seq_len], v[:seq_len]


# --------------------------------------------------------------------------
# Scores, whole-sequence output, partition partials, merge
# --------------------------------------------------------------------------

def sequence_logits(q: np.ndarray, k: np.ndarray, scale: float,
                    alibi_slopes: Optional[np.ndarray], window_left: int = -1,
                    soft_cap: float = 0.0) -> np.ndarray:
    """Scaled logits s[h, t] for one sequence.

    q [H, D] float64, k [L, Hkv, D] float64.  Query head h reads KV head
    h // (H / Hkv) (V2 page, GQA expansion by repeat_interleave).
    s[h, t] = scale * sum_d q[h, d] k[t, kv(h), d]  +  slope[h] * t
    (V2 page, Phase 1: scores, then the ALiBi bias with absolute positions).
    With soft_cap c > 0 the scaled dot product is replaced by c * tanh(. / c)
    before the bias; with window_left W >= 0 the keys t < L - 1 - W get -inf
    (the decode configuration fields of the dispatch page, read as described
    in the module docstring).
    """
    num_heads = q.shape[0]
    seq_len, hkv, _ = k.shape
    group = num_heads // hkv
    s = np.empty((num_heads, seq_len))
    for h in range(num_heads):
        s[h] = (k[:, h // group, :] @ q[h]) * scale
    if soft_cap > 0.0:
        s = soft_cap * np.tanh(s / soft_cap)
    if alibi_slopes is not None:
        positions = np.arange(seq_len, dtype=np.float64)
        s = s + np.asarray(alibi_slopes, dtype=np.float64)[:, None] * positions[None, :]
    if window_left >= 0:
        s[:, :max(0, seq_len - 1 - window_left)] = -np.inf
    return s


def _weighted_values(w: np.ndarray, v: np.ndarray) -> np.ndarray:
    """sum_t w[h, t] * v[t, kv(h), :] for every query head h -> [H, D]."""
    num_heads = w.shape[0]
    group = num_heads // v.shape[1]
    return np.stack([w[h] @ v[:, h // group, :] for h in range(num_heads)])


def softmax_output(s: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Whole-sequence softmax attention output (the v1 result).

    out[h] = sum_t w[h,t] v[t, kv(h)] / sum_t w[h,t],  w = exp(s - max_t s)
    (dispatch page, PyTorch decode fallback: softmax(scores) . V).
    """
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return _weighted_values(w, v) / w.sum(axis=1)[:, None]


def partition_partials(s: np.ndarray, v: np.ndarray, max_num_partitions: int,
                       partition_size: int = PARTITION_SIZE):
    """Phase 1 of the V2 page: statistics and output of every partition.

    For partition p covering tokens T_p = [p*PS, min((p+1)*PS, L)):
      m_p = max_{t in T_p} s[h, t]                      (max_logits)
      S_p = sum_{t in T_p} exp(s[h, t] - m_p)           (exp_sums)
      O_p = sum_{t in T_p} exp(s[h, t] - m_p) v_t / S_p  (tmp_output, normalised)
    Partitions P_s <= p < max_num_partitions are padding: -inf, 0, 0; so is a
    partition in which no key is visible (all its logits -inf: before a
    sliding window).
    Returns (max_logits [H, P], exp_sums [H, P], tmp_out [H, P, D]).
    """
    num_heads, seq_len = s.shape
    head_size = v.shape[2]
    n_part = num_partitions(seq_len, partition_size)
    assert n_part <= max_num_partitions
    max_logits = np.full((num_heads, max_num_partitions), -np.inf)
    exp_sums = np.zeros((num_heads, max_num_partitions))
    tmp_out = np.zeros((num_heads, max_num_partitions, head_size))
    for p in range(n_part):
        start = p * partition_size
        end = min(start + partition_size, seq_len)
        sp = s[:, start:end]
        m_p = sp.max(axis=1)
        if np.all(np.isneginf(m_p)):
            continue
        e = np.exp(sp - m_p[:, None])
        s_p = e.sum(axis=1)
        max_logits[:, p] = m_p
        exp_sums[:, p] = s_p
        tmp_out[:, p, :] = _weighted_values(e, v[start:end]) / s_p[:, None]
    return max_logits, exp_sums, tmp_out


def merge_partials(max_logits: np.ndarray, exp_sums: np.ndarray,
                   tmp_out: np.ndarray, n_part: int) -> np.ndarray:
    """Phase 2 of the V2 page: log-sum-exp merge of the first n_part partitions.

      M   = max_p m_p
      r_p = exp(m_p - M) * S_p
      out = sum_p (r_p / sum_q r_q) * O_p
    """
    m = max_logits[:, :n_part]
    big_m = m.max(axis=1)
    r = np.exp(m - big_m[:, None]) * exp_sums[:, :n_part]
    weights = r / r.sum(axis=1)[:, None]
    return np.einsum("hp,hpd->hd", weights, tmp_out[:, :n_part, :])


# --------------------------------------------------------------------------
# Whole batch
# --------------------------------------------------------------------------

def paged_attention(query_raw: np.ndarray, key_cache_raw: np.ndarray,
                    value_cache_raw: np.ndarray, block_tables: np.ndarray,
                    seq_lens: np.ndarray, scale: float, *, q_kind: str,
                    kv_kind: str, k_scale: float = 1.0, v_scale: float = 1.0,
                    alibi_slopes: Optional[np.ndarray] = None,
                    max_num_partitions: Optional[int] = None,
                    partition_size: int = PARTITION_SIZE,
                    seqs: Optional[list] = None,
                    check_merge: bool = True, window_left: int = -1,
                    soft_cap: float = 0.0) -> Dict[str, np.ndarray]:
    """Reference v1 output and v2 partials/merged output for a decode batch.

    query_raw [B, H, D] and the caches are raw storage (see decode_storage);
    block_tables int32 [B, max_blocks_per_seq]; seq_lens int [B].
    ``seqs`` restricts the work to those batch rows (others stay zero /
    padding).  ``window_left`` / ``soft_cap``: see sequence_logits.  Returns a dict of float64 arrays:
      out_v1 [B, H, D], out_v2 [B, H, D], max_logits [B, H, P],
      exp_sums [B, H, P], tmp_out [B, H, P, D].
    With ``check_merge`` the merged v2 output is asserted equal to the
    whole-sequence softmax to 1e-10 relative (the V2 page's claim that the
    log-sum-exp reduction is equivalent to the full softmax).
    """
    num_seqs, num_heads, head_size = query_raw.shape
    block_size = key_cache_raw.shape[3]
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if max_num_partitions is None:
        max_num_partitions = max(1, num_partitions(int(seq_lens.max(initial=0)), partition_size))
    q_all = decode_storage(query_raw, q_kind)
    out_v1 = np.zeros((num_seqs, num_heads, head_size))
    out_v2 = np.zeros((num_seqs, num_heads, head_size))
    max_logits = np.full((num_seqs, num_heads, max_num_partitions), -np.inf)
    exp_sums = np.zeros((num_seqs, num_heads, max_num_partitions))
    tmp_out = np.zeros((num_seqs, num_heads, max_num_partitions, head_size))
    rows = range(num_seqs) if seqs is None else seqs
    for b in rows:
        seq_len = int(seq_lens[b])
        if seq_len == 0:
            continue
        n_logical = (seq_len + block_size - 1) // block_size
        phys = np.asarray(block_tables[b, :n_logical], dtype=np.int64)
        k_pool = decode_storage(key_cache_raw[phys], kv_kind) * k_scale
        v_pool = decode_storage(value_cache_raw[phys], kv_kind) * v_scale
        k, v = gather_sequence(k_pool, v_pool, np.arange(n_logical), seq_len, block_size)
        s = sequence_logits(q_all[b], k, scale, alibi_slopes, window_left, soft_cap)
        out_v1[b] = softmax_output(s, v)
        ml, es, to = partition_partials(s, v, max_num_partitions, partition_size)
        max_logits[b], exp_sums[b], tmp_out[b] = ml, es, to
        out_v2[b] = merge_partials(ml, es, to, num_partitions(seq_len, partition_size))
        if check_merge:
            denom = max(np.abs(out_v1[b]).max(), 1e-300)
            assert np.abs(out_v2[b] - out_v1[b]).max() <= 1e-10 * denom, \
                "log-sum-exp merge disagrees with the whole-sequence softmax"
    return {"out_v1": out_v1, "out_v2": out_v2, "max_logits": max_logits,
            "exp_sums": exp_sums, "tmp_out": tmp_out}


# --------------------------------------------------------------------------
# v1/v2 dispatch rule (host-side definition, for pinning the library's mirror)
# --------------------------------------------------------------------------

def page_should_use_v2(seq_len: int, num_kv_heads: int, sm_count: int,
                       threshold_factor: int = 2,
                       partition_size: int = PARTITION_SIZE) -> bool:
    """The dispatch page's rule ``should_use_paged_v2``: with
    tiles = num_kv_heads * ceil(seq_len / partition_size), use v2 iff
    tiles > threshold_factor * sm_count."""
    tiles = num_kv_heads * num_partitions(seq_len, partition_size)
    return tiles > threshold_factor * sm_count
