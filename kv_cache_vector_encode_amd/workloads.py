"""Seeded synthetic workloads (shapes, value distributions, paging).

This module generates inputs only: random keys, values, queries, slot
mappings and block tables.  It holds none of the codec's arithmetic, so both
the HIP path and the CPU oracle may consume what it produces.

Distributions (the pages measure on LongBench / needle-in-a-haystack /
WikiText-2 / C4 with trained models; these seeded inputs stand in for them):
  * outlier keys: per KV head h a per-channel log-normal scale
    lambda_{h,j} = exp(N(0,1)) and two distinct outlier channels scaled x30;
    K = N(0,1) * lambda * (30 on outlier channels), rounded to bf16;
  * values and queries: N(0,1), rounded to bf16;
  * the tiny case: fp32 keys N(0,1) with two channels scaled x30, one fp32
    query N(0,1);
  * paging: physical blocks are a seeded permutation of range(num_blocks)
    dealt to sequences in order (non-contiguous block tables).
Every stream comes from its own ``numpy.random.SeedSequence(seed).spawn``
child (PCG64), so each array is reproducible on its own.
"""

from __future__ import annotations

import dataclasses

import numpy as np

BLOCK = 16

# stream indices of SeedSequence(seed).spawn(N_STREAMS)
_S_K, _S_V, _S_Q, _S_SCALE, _S_OUTLIER, _S_PERM, _S_SPARE = range(7)
N_STREAMS = 7


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_seqs: int
    seq_len: int
    num_kv_heads: int
    num_q_heads: int
    bits_k: int
    bits_v: int          # 0 => keys-only cache
    qjl: bool
    key_dist: str        # "outlier" | "tiny"
    in_dtype: str        # "bf16" | "f32"
    head_dim: int = 128
    rot_seed: int = 42   # seed of R (the pages' example uses hadamard_seed=42)
    qjl_seed: int = 43   # seed of the independent R'

    @property
    def tokens(self) -> int:
        return self.num_seqs * self.seq_len

    @property
    def blocks_per_seq(self) -> int:
        return -(-self.seq_len // BLOCK)

    @property
    def num_blocks(self) -> int:
        return self.num_seqs * self.blocks_per_seq

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five synthetic configurations.
TINY = Workload("tiny_4096x128_f32_b4", 0, 1, 4096, 1, 1, 4, 0, False, "tiny", "f32")
DECODE_32K = Workload("decode_1x32768_h8_gqa8_b4", 2, 1, 32768, 8, 64, 4, 4, False, "outlier", "bf16")
LLAMA70B_128K = Workload("llama70b_4x131072_h8_gqa8_b3", 3, 4, 131072, 8, 64, 3, 3, False, "outlier", "bf16")
SWEEP_64K = Workload("sweep_16h_65536_keys", 4, 1, 65536, 16, 16, 4, 0, False, "outlier", "bf16")
PREFILL_16x8K = Workload("prefill_16x8192_h8_gqa8_b4", 5, 16, 8192, 8, 64, 4, 4, False, "outlier", "bf16")

CONFIGS = {w.name: w for w in (TINY, DECODE_32K, LLAMA70B_128K, SWEEP_64K, PREFILL_16x8K)}


def _streams(seed: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(N_STREAMS)]


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def key_channel_scales(w: Workload) -> np.ndarray:
    """Per (KV head, channel) multiplier: log-normal scale x (30 on the two
    outlier channels).  Shape (num_kv_heads, head_dim), float64."""
    st = _streams(w.seed)
    d, H = w.head_dim, w.num_kv_heads
    if w.key_dist == "tiny":
        m = np.ones((H, d))
        for h in range(H):
            m[h, st[_S_OUTLIER].choice(d, 2, replace=False)] = 30.0
        return m
    lam = np.exp(st[_S_SCALE].standard_normal((H, d)))
    for h in range(H):
        lam[h, st[_S_OUTLIER].choice(d, 2, replace=False)] *= 30.0
    return lam


def _normal_rows(rng_seed_seq, start: int, count: int, width: int) -> np.ndarray:
    # rows [start, start+count) of an (infinite) N(0,1) matrix of row width
    # ``width``; each row block of 4096 rows has its own child seed, so any
    # sub-range is reproducible without generating the prefix.
    out = np.empty((count, width), dtype=np.float32)
    CH = 4096
    r = start
    while r < start + count:
        blk = r // CH
        rng = np.random.default_rng(np.random.SeedSequence(entropy=rng_seed_seq, spawn_key=(blk,)))
        rows = rng.standard_normal((CH, width), dtype=np.float32)
        lo = r - blk * CH
        n = min(CH - lo, start + count - r)
        out[r - start:r - start + n] = rows[lo:lo + n]
        r += n
    return out


def _stream_entropy(w: Workload, which: int) -> int:
    return int(np.random.SeedSequence(w.seed).spawn(N_STREAMS)[which].generate_state(1, np.uint64)[0])


def keys(w: Workload, tok_start: int = 0, tok_count: int | None = None):
    """Keys for global tokens [tok_start, tok_start + tok_count), all heads.

    Returns (array_for_device, exact_float64) where array_for_device is
    uint16 bf16 bits (bf16 workloads) or float32 (the tiny fp32 case), shape
    (tok_count, num_kv_heads, head_dim)."""
    if tok_count is None:
        tok_count = w.tokens - tok_start
    H, d = w.num_kv_heads, w.head_dim
    z = _normal_rows(_stream_entropy(w, _S_K), tok_start * H, tok_count * H, d)
    z = z.reshape(tok_count, H, d).astype(np.float64) * key_channel_scales(w)[None]
    z32 = z.astype(np.float32)
    if w.in_dtype == "f32":
        return z32, z32.astype(np.float64)
    b = bf16_bits(z32)
    return b, bf16_to_f64(b)


def values(w: Workload, tok_start: int = 0, tok_count: int | None = None):
    if tok_count is None:
        tok_count = w.tokens - tok_start
    H, d = w.num_kv_heads, w.head_dim
    z32 = _normal_rows(_stream_entropy(w, _S_V), tok_start * H, tok_count * H, d).reshape(tok_count, H, d)
    if w.in_dtype == "f32":
        return z32, z32.astype(np.float64)
    b = bf16_bits(z32)
    return b, bf16_to_f64(b)


def queries(w: Workload, num_seqs: int | None = None):
    """Queries (num_seqs, num_q_heads, head_dim): N(0,1), bf16 or fp32."""
    n = w.num_seqs if num_seqs is None else num_seqs
    z32 = _normal_rows(_stream_entropy(w, _S_Q), 0, n * w.num_q_heads, w.head_dim)
    z32 = z32.reshape(n, w.num_q_heads, w.head_dim)
    if w.in_dtype == "f32":
        return z32, z32.astype(np.float64)
    b = bf16_bits(z32)
    return b, bf16_to_f64(b)


def block_tables(w: Workload) -> np.ndarray:
    """int32 (num_seqs, blocks_per_seq): a seeded permutation of the physical
    blocks dealt to sequences in order."""
    perm = _streams(w.seed)[_S_PERM].permutation(w.num_blocks).astype(np.int32)
    return perm.reshape(w.num_seqs, w.blocks_per_seq)


def slot_mapping(w: Workload) -> np.ndarray:
    """int32 (tokens,): slot = physical_block * 16 + row for every token
    (token t of sequence s sits at logical block t // 16, row t % 16)."""
    bt = block_tables(w)
    t = np.arange(w.seq_len)
    per_seq = bt[:, t // BLOCK] * BLOCK + (t % BLOCK)[None, :]
    return per_seq.reshape(-1).astype(np.int32)


def seq_lens(w: Workload) -> np.ndarray:
    return np.full(w.num_seqs, w.seq_len, dtype=np.int32)
