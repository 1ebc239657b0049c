"""Seeded synthetic inputs for paged decode attention.

This module only draws inputs: sequence lengths, a shuffled page pool with its
block table, the slot of every token, and q / k / v rows as BF16 bit patterns.
It holds none of the attention, softmax, quantization or cache-layout
arithmetic; both the CPU oracle (``oracle/``) and the HIP path consume what it
returns, and neither is imported here.

Workloads (shapes from the problem statement of the paged decode launchers on
the metrale ``prefill_attn_b.rs`` page and the AstrAI ``csrc/tests`` commit
log; values are i.i.d. normal draws, because no dataset is involved):

* ``tiny``     2 seqs (lens 17, 40), 4 q / 2 kv heads, head_dim 64, block 16,
               block table = a random permutation of 8 pages laid out 2 x 4.
* ``llama8b``  32 seqs, lens uniform in [512, 4096], 32 q / 8 kv heads,
               head_dim 128, block 16, shuffled page pool.
* ``b1_<ctx>`` 1 seq of ctx tokens (128, 1K..32K), 32 q / 8 kv heads, head_dim 128.
* ``fp8``      64 seqs, lens uniform in [1K, 8K], 16 q / 8 kv heads,
               head_dim 256, sliding window 4096, K/V ~ N(0, 2^2).
* ``nvfp4``    16 seqs, lens uniform in [2K, 16K], 16 q / 2 kv heads,
               head_dim 512.

Draw order for a seed: seq_lens, page permutation, q, k, v (then the optional
"new token" rows used by a decode step).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

__all__ = [
    "DecodeWorkload",
    "WORKLOADS",
    "make_workload",
    "bf16_bits_from_f32",
    "workload_names",
    "query_block",
]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to BF16 (round-to-nearest-even, via torch's cast)
    and return the 16-bit patterns as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class DecodeWorkload:
    name: str
    kv_dtype: str            # "bf16" | "fp8" | "nvfp4"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    max_blocks_per_seq: int
    sliding_window: int
    scale: np.float32        # softmax scale applied after the q.k dot
    seq_lens: np.ndarray     # int32 [B]
    block_tables: np.ndarray  # int32 [B, max_blocks_per_seq]
    num_pages: int           # physical pages in the pool
    q_bits: np.ndarray       # uint16 [B, Hq, D]    (BF16 patterns)
    k_bits: np.ndarray       # uint16 [T, Hkv, D]   token-major, all tokens of all seqs
    v_bits: np.ndarray       # uint16 [T, Hkv, D]
    slot_mapping: np.ndarray  # int32 [T]  slot = page * block_size + offset
    token_seq: np.ndarray    # int32 [T]  sequence of token t
    token_pos: np.ndarray    # int32 [T]  position of token t in its sequence
    num_splits: tuple = ()   # split counts the parity tests exercise

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def last_token_index(self) -> np.ndarray:
        """Index into k_bits/v_bits of the last token of every sequence (the
        token a decode step appends); -1 for empty sequences."""
        ends = np.cumsum(self.seq_lens.astype(np.int64)) - 1
        ends[self.seq_lens == 0] = -1
        return ends


# name -> (kv_dtype, B, Hq, Hkv, D, bs, lens spec, window, kv sigma, seed, splits)
_SPECS = {
    "tiny": ("bf16", 2, 4, 2, 64, 16, ("fixed", (17, 40)), 0, 1.0, 0, (1, 3)),
    "llama8b": ("bf16", 32, 32, 8, 128, 16, ("uniform", 512, 4096), 0, 1.0, 1, ()),
    "fp8": ("fp8", 64, 16, 8, 256, 16, ("uniform", 1024, 8192), 4096, 2.0, 3, ()),
    "nvfp4": ("nvfp4", 16, 16, 2, 512, 16, ("uniform", 2048, 16384), 0, 1.0, 4, ()),
}
for _ctx in (1024, 4096, 8192, 16384, 32768):
    _SPECS[f"b1_{_ctx // 1024}k"] = ("bf16", 1, 32, 8, 128, 16, ("fixed", (_ctx,)), 0, 1.0, 2, ())
_SPECS["b1_128"] = ("bf16", 1, 32, 8, 128, 16, ("fixed", (128,)), 0, 1.0, 2, ())

WORKLOADS = dict(_SPECS)


def workload_names():
    return list(_SPECS)


def make_workload(
    name: str,
    *,
    seed: Optional[int] = None,
    num_seqs: Optional[int] = None,
    kv_dtype: Optional[str] = None,
    lens: Optional[tuple] = None,
    extra_pages: int = 8,
    identity_pages: bool = False,
    with_kv: bool = True,
    num_q_heads: Optional[int] = None,
    num_kv_heads: Optional[int] = None,
    head_dim: Optional[int] = None,
    block_size: Optional[int] = None,
    sliding_window: Optional[int] = None,
    sigma: Optional[float] = None,
) -> DecodeWorkload:
    """Draw a workload. ``num_seqs`` keeps the first sequence lengths of the
    full draw and draws everything else at that smaller size (a sample of the
    same distribution, not a slice of the full run's values); ``lens``
    overrides the lengths; ``identity_pages`` lays the pool out in order
    instead of shuffling it; ``with_kv=False`` skips K/V. The shape
    arguments override the named workload's heads, head_dim, block size,
    window and K/V standard deviation."""
    spec = _SPECS[name]
    (dt, B, Hq, Hkv, D, bs, lens_spec, window, sig, seed0, splits) = spec
    dt = kv_dtype or dt
    Hq = num_q_heads or Hq
    Hkv = num_kv_heads or Hkv
    D = head_dim or D
    bs = block_size or bs
    window = window if sliding_window is None else sliding_window
    sigma = sig if sigma is None else sigma
    rng = np.random.default_rng(seed0 if seed is None else seed)

    if lens is not None:
        seq_lens = np.asarray(lens, dtype=np.int64)
        B = len(seq_lens)
    elif lens_spec[0] == "fixed":
        seq_lens = np.asarray(lens_spec[1], dtype=np.int64)
    else:
        seq_lens = rng.integers(lens_spec[1], lens_spec[2], size=B, endpoint=True)
    if num_seqs is not None:
        seq_lens = seq_lens[:num_seqs]
        B = num_seqs

    pages_per_seq = (seq_lens + bs - 1) // bs
    if name == "tiny" and lens is None and num_seqs is None and block_size is None:
        # 8 physical pages laid out as a 2 x 4 table; entries past a
        # sequence's last page are valid page ids that are never read.
        max_blocks = 4
        num_pages = 8
        perm = np.arange(num_pages) if identity_pages else rng.permutation(num_pages)
        block_tables = perm.reshape(B, max_blocks).astype(np.int32)
    else:
        max_blocks = int(max(1, pages_per_seq.max(initial=1)))
        if lens_spec[0] == "uniform" and lens is None and block_size is None:
            max_blocks = int((lens_spec[2] + bs - 1) // bs)
        used = int(pages_per_seq.sum())
        num_pages = used + extra_pages
        perm = np.arange(num_pages) if identity_pages else rng.permutation(num_pages)
        block_tables = np.zeros((B, max_blocks), dtype=np.int32)
        cur = 0
        for b in range(B):
            n = int(pages_per_seq[b])
            block_tables[b, :n] = perm[cur:cur + n]
            cur += n

    q_bits = bf16_bits_from_f32(rng.standard_normal((B, Hq, D), dtype=np.float32))

    T = int(seq_lens.sum())
    token_seq = np.repeat(np.arange(B, dtype=np.int32), seq_lens)
    starts = np.concatenate([[0], np.cumsum(seq_lens)[:-1]]).astype(np.int64)
    token_pos = (np.arange(T, dtype=np.int64) - np.repeat(starts, seq_lens)).astype(np.int32)
    pages = block_tables[token_seq, token_pos // bs].astype(np.int64)
    slot_mapping = (pages * bs + token_pos % bs).astype(np.int32)

    if with_kv:
        k_bits = bf16_bits_from_f32(rng.standard_normal((T, Hkv, D), dtype=np.float32) * np.float32(sigma))
        v_bits = bf16_bits_from_f32(rng.standard_normal((T, Hkv, D), dtype=np.float32) * np.float32(sigma))
    else:
        k_bits = np.zeros((0, Hkv, D), np.uint16)
        v_bits = np.zeros((0, Hkv, D), np.uint16)

    return DecodeWorkload(
        name=name, kv_dtype=dt, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, block_size=bs, max_blocks_per_seq=max_blocks,
        sliding_window=int(window), scale=np.float32(1.0 / np.sqrt(D)),
        seq_lens=seq_lens.astype(np.int32), block_tables=block_tables,
        num_pages=int(num_pages), q_bits=q_bits, k_bits=k_bits, v_bits=v_bits,
        slot_mapping=slot_mapping, token_seq=token_seq, token_pos=token_pos,
        num_splits=tuple(splits),
    )


def query_block(w: DecodeWorkload, q_len: int, seed: int = 0) -> np.ndarray:
    """q_len query tokens per sequence for multi-token attention over the
    workload's cache (a speculative-verify or chunked-prefill block): BF16
    patterns [B, q_len, Hq, D] of N(0, 1) draws, from a generator of its own
    (seeded by ``seed`` and q_len) so the workload's other draws are
    unchanged."""
    rng = np.random.default_rng([seed, q_len, 7])
    x = rng.standard_normal((w.num_seqs, q_len, w.num_q_heads, w.head_dim), dtype=np.float32)
    return bf16_bits_from_f32(x)
