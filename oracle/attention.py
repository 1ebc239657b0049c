"""Paged decode attention in float64, by the definition.

One query token per sequence attends over that sequence's keys, which sit in
fixed-size pages found through the block table [metrale: paged decode
launchers' doc comments]. Query head h reads kv head h / (Hq/Hkv), consecutive
q heads sharing one kv head (R16) [AstrAI log: q_head/kv_head divisibility
check]. The logit is the q.k dot product multiplied by the softmax scale after
the dot [AstrAI log: numerics bullets]. With a sliding window W > 0 the
sequence attends to its last W keys, the current one included (R17); W = 0
means no window. An empty key range gives a zero output (R19).

The split-KV form [metrale: paged_decode_attn_splitk_nvfp4 and
paged_decode_attn_reduce_fp8: per split a partial output plus the softmax
state (m, l), then a combine into the output; AstrAI log: split-KV decode with
one shared combine]: the pages of the attended range are cut into chunks of
``c`` pages, c = ceil(P / S) for a page bound P that the launch knows (R20);
split i takes chunk i. Each split keeps o_i = sum p v / l_i (normalized),
m_i = its largest scaled logit, l_i = sum exp(s - m_i); an empty split has
m = -inf, l = 0, o = 0. The combine weighs split i by l_i * exp(m_i - M), M
the largest m_i of a non-empty split, and divides by max(sum of weights,
1e-20) [AstrAI log: divide-by-zero guard].
"""
from __future__ import annotations

import math

import numpy as np

from .cache import CacheGeometry, read_kv_rows
from .formats import bf16_to_f64, e4m3_decode


def window_start(seq_len: int, sliding_window: int) -> int:
    """First attended position: L - W when a window W > 0 is shorter than L."""
    if sliding_window > 0 and seq_len > sliding_window:
        return seq_len - sliding_window
    return 0


def attention_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of q [Hq, D] over K, V [n, Hkv, D], float64."""
    Hq, D = q.shape
    n, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if n == 0:
        return out
    for h in range(Hq):
        g = h // G
        s = (K[:, g, :] @ q[h]) * float(scale)
        p = np.exp(s - s.max())
        out[h] = (p @ V[:, g, :]) / p.sum()
    return out


def _q_rows(q_bits, b, Hq, D, q_stride):
    flat = np.asarray(q_bits, dtype=np.uint16).reshape(-1)
    idx = b * q_stride + np.arange(Hq)[:, None] * D + np.arange(D)[None, :]
    return bf16_to_f64(flat[idx])


def _seq_kv(geom, k_cache, v_cache, block_tables, b, lo, L, k_scale, v_scale):
    j = np.arange(lo, L, dtype=np.int64)
    bs = geom.block_size
    pages = np.asarray(block_tables)[b, j // bs].astype(np.int64)
    offs = j % bs
    K = read_kv_rows(geom, k_cache, pages, offs, k_scale)
    V = read_kv_rows(geom, v_cache, pages, offs, v_scale)
    return K, V


def paged_decode_attention(geom: CacheGeometry, q_bits, k_cache, v_cache, block_tables,
                           seq_lens, num_q_heads, scale, q_stride=None,
                           sliding_window=0, k_scale=1.0, v_scale=1.0, seqs=None) -> np.ndarray:
    """Exact output [len(seqs), Hq, D] (float64) of paged decode attention:
    gather the attended pages into contiguous K/V, dequantize, softmax."""
    D = geom.head_dim
    Hq = num_q_heads
    q_stride = Hq * D if q_stride is None else q_stride
    seq_lens = np.asarray(seq_lens).reshape(-1)
    seqs = range(len(seq_lens)) if seqs is None else seqs
    out = []
    for b in seqs:
        L = int(seq_lens[b])
        lo = window_start(L, sliding_window)
        K, V = _seq_kv(geom, k_cache, v_cache, block_tables, b, lo, L, k_scale, v_scale)
        out.append(attention_rows(_q_rows(q_bits, b, Hq, D, q_stride), K, V, scale))
    return np.stack(out) if out else np.zeros((0, Hq, D))


def split_page_bound(max_blocks_per_seq: int, block_size: int, sliding_window: int) -> int:
    """Most pages one sequence's attended range can touch: the block-table
    width, or, with a window of W keys, (W + block_size - 2) // block_size + 1
    when that is smaller (W keys starting mid-page)."""
    bound = max_blocks_per_seq
    if sliding_window > 0:
        bound = min(bound, (sliding_window + block_size - 2) // block_size + 1)
    return max(1, bound)


def split_partials(geom: CacheGeometry, q_bits, k_cache, v_cache, block_tables, seq_lens,
                   num_q_heads, scale, num_splits, max_blocks_per_seq, q_stride=None,
                   sliding_window=0, k_scale=1.0, v_scale=1.0):
    """Per-split partials: o [B, Hq, S, D] (normalized), m [B, Hq, S], l [B, Hq, S]."""
    D, bs = geom.head_dim, geom.block_size
    Hq = num_q_heads
    q_stride = Hq * D if q_stride is None else q_stride
    seq_lens = np.asarray(seq_lens).reshape(-1)
    B, S = len(seq_lens), int(num_splits)
    c = math.ceil(split_page_bound(max_blocks_per_seq, bs, sliding_window) / S)
    o = np.zeros((B, Hq, S, D))
    m = np.full((B, Hq, S), -np.inf)
    l = np.zeros((B, Hq, S))
    for b in range(B):
        L = int(seq_lens[b])
        lo = window_start(L, sliding_window)
        p0, pend = lo // bs, (L + bs - 1) // bs
        q = _q_rows(q_bits, b, Hq, D, q_stride)
        G = Hq // geom.num_kv_heads
        for i in range(S):
            t0 = max(lo, (p0 + i * c) * bs)
            t1 = min(L, min(p0 + (i + 1) * c, pend) * bs)
            if t1 <= t0:
                continue
            K, V = _seq_kv(geom, k_cache, v_cache, block_tables, b, t0, t1, k_scale, v_scale)
            for h in range(Hq):
                s = (K[:, h // G, :] @ q[h]) * float(scale)
                m[b, h, i] = s.max()
                p = np.exp(s - m[b, h, i])
                l[b, h, i] = p.sum()
                o[b, h, i] = (p @ V[:, h // G, :]) / l[b, h, i]
    return o, m, l


def combine_partials(o: np.ndarray, m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """Merge split partials [B, Hq, S, ...] into the output [B, Hq, D]."""
    live = l > 0
    M = np.where(live, m, -np.inf).max(axis=-1, initial=-np.inf)
    safe_M = np.where(np.isfinite(M), M, 0.0)
    w = np.where(live, l * np.exp(np.where(live, m, 0.0) - safe_M[..., None]), 0.0)
    num = (w[..., None] * o).sum(axis=-2)
    den = np.maximum(w.sum(axis=-1), 1e-20)
    return num / den[..., None]


def query_range(seq_len: int, q_len: int, i: int, causal: bool, sliding_window: int):
    """Keys [lo, hi) that query token i of a q_len-token block attends.

    Multi-token paged attention (chunked prefill, speculative verify) over the
    same block table [pegainfer #1008: the paged prefill launch body; AstrAI
    log: unified causal_offset, -1 = off, >= 0 = the first query position]:
    the block's tokens are the sequence's newest, already in the cache, so in
    a batch of ragged lengths the first query position of sequence b is
    L_b - q_len and token i sits at p = L - q_len + i (R26). Causal: keys
    0..p, the last W of them with a window W > 0. Not causal (the offset -1):
    every token attends what a one-token decode of the sequence would,
    [window_start(L, W), L). A token at a negative position attends nothing."""
    if not causal:
        return window_start(seq_len, sliding_window), seq_len
    p = seq_len - q_len + i
    hi = max(p + 1, 0)
    lo = max(0, p + 1 - sliding_window) if sliding_window > 0 else 0
    return min(lo, hi), hi


def _prefill_q_rows(q_bits, b, i, Hq, D, q_stride, q_token_stride):
    flat = np.asarray(q_bits, dtype=np.uint16).reshape(-1)
    idx = b * q_stride + i * q_token_stride + np.arange(Hq)[:, None] * D + np.arange(D)[None, :]
    return bf16_to_f64(flat[idx])


def paged_prefill_attention(geom: CacheGeometry, q_bits, k_cache, v_cache, block_tables,
                            seq_lens, num_q_heads, q_len, scale, causal=True, q_stride=None,
                            q_token_stride=None, sliding_window=0, k_scale=1.0, v_scale=1.0,
                            seqs=None, return_state=False):
    """Exact output [len(seqs), q_len, Hq, D] (float64) of multi-token paged
    attention: for each sequence and each of its q_len query tokens, gather
    the token's key range (``query_range``) through the block table,
    dequantize, softmax. q token i of sequence b is the BF16 row block at
    b * q_stride + i * q_token_stride (elements; defaults: contiguous
    [B, q_len, Hq, D]). With ``return_state`` also the largest scaled logit m
    and the sum l of exp(s - m) of every query row (-inf and 0 when the row
    attends nothing)."""
    D = geom.head_dim
    Hq = num_q_heads
    G = Hq // geom.num_kv_heads
    q_token_stride = Hq * D if q_token_stride is None else q_token_stride
    q_stride = q_len * q_token_stride if q_stride is None else q_stride
    seq_lens = np.asarray(seq_lens).reshape(-1)
    seqs = list(range(len(seq_lens)) if seqs is None else seqs)
    out = np.zeros((len(seqs), q_len, Hq, D))
    m = np.full((len(seqs), q_len, Hq), -np.inf)
    l = np.zeros((len(seqs), q_len, Hq))
    for r, b in enumerate(seqs):
        L = int(seq_lens[b])
        for i in range(q_len):
            lo, hi = query_range(L, q_len, i, causal, sliding_window)
            K, V = _seq_kv(geom, k_cache, v_cache, block_tables, b, lo, hi, k_scale, v_scale)
            q = _prefill_q_rows(q_bits, b, i, Hq, D, q_stride, q_token_stride)
            out[r, i] = attention_rows(q, K, V, scale)
            if return_state and hi > lo:
                for h in range(Hq):
                    s = (K[:, h // G, :] @ q[h]) * float(scale)
                    m[r, i, h] = s.max()
                    l[r, i, h] = np.exp(s - s.max()).sum()
    if return_state:
        return out, m, l
    return out


def contiguous_kv_rows(fmt: str, data, b: int, lo: int, hi: int, num_kv_heads: int,
                       head_dim: int, strides, scale=1.0) -> np.ndarray:
    """Rows [hi - lo, Hkv, D] (float64, exact) of keys lo .. hi-1 of sequence b
    in a contiguous K or V tensor (no block table) [AstrAI log: the ContigKV
    source policy; stride-based Q/KV/O addressing]: element
    b*strides[0] + j*strides[1] + h*strides[2] + d. BF16 bits, or E4M3 codes
    times the per-tensor scale."""
    flat = np.asarray(data).reshape(-1)
    j = np.arange(lo, hi, dtype=np.int64)[:, None, None]
    h = np.arange(num_kv_heads, dtype=np.int64)[None, :, None]
    d = np.arange(head_dim, dtype=np.int64)[None, None, :]
    idx = b * int(strides[0]) + j * int(strides[1]) + h * int(strides[2]) + d
    if fmt == "bf16":
        return bf16_to_f64(flat[idx])
    if fmt == "fp8":
        return e4m3_decode(flat[idx]) * float(np.float32(scale))
    raise ValueError(f"contiguous K/V rows are BF16 or FP8, not {fmt}")


def contiguous_attention(fmt: str, q_bits, k_data, v_data, seq_lens, num_q_heads: int,
                         num_kv_heads: int, head_dim: int, q_len: int, scale, q_strides,
                         k_strides, v_strides, causal=True, sliding_window=0, k_scale=1.0,
                         v_scale=1.0, seqs=None) -> np.ndarray:
    """Exact output [len(seqs), q_len, Hq, D] (float64) of multi-token
    attention over contiguous K/V tensors: q token i of sequence b, head h at
    b*q_strides[0] + i*q_strides[1] + h*q_strides[2]; the keys each token
    attends as in ``query_range``; softmax as in ``attention_rows``."""
    D, Hq = head_dim, num_q_heads
    qflat = np.asarray(q_bits, dtype=np.uint16).reshape(-1)
    seq_lens = np.asarray(seq_lens).reshape(-1)
    seqs = list(range(len(seq_lens)) if seqs is None else seqs)
    out = np.zeros((len(seqs), q_len, Hq, D))
    hq = np.arange(Hq, dtype=np.int64)[:, None]
    d = np.arange(D, dtype=np.int64)[None, :]
    for r, b in enumerate(seqs):
        L = int(seq_lens[b])
        for i in range(q_len):
            lo, hi = query_range(L, q_len, i, causal, sliding_window)
            K = contiguous_kv_rows(fmt, k_data, b, lo, hi, num_kv_heads, D, k_strides, k_scale)
            V = contiguous_kv_rows(fmt, v_data, b, lo, hi, num_kv_heads, D, v_strides, v_scale)
            q = bf16_to_f64(qflat[b * int(q_strides[0]) + i * int(q_strides[1]) +
                                  hq * int(q_strides[2]) + d])
            out[r, i] = attention_rows(q, K, V, scale)
    return out
