"""Paged KV caches: layout, the slot-mapping cache write and the BF16 absmax.

Layouts (K and V are separate pools with the same layout):

* BF16: ``[pages, block_size, kv_heads, head_dim]`` elements, page stride
  block_size * kv_heads * head_dim [metrale: paged_decode_attn_splitk_bf16,
  which states this order and has the kernel derive the page stride].
* FP8: the same index order in bytes, consecutive physical pages
  ``cache_stride`` bytes apart (R11) [metrale: paged_decode_attn_splitk_fp8
  takes the stride].
* NVFP4: page p starts at p * block_stride_bytes; its first
  data_section_bytes hold E2M1 codes, the E4M3 scales follow
  [metrale: reshape_and_cache_nvfp4]. Within a page (R12): element d of
  (offset o, head h) is the nibble of byte (o*Hkv + h)*D/2 + d/2, the low
  nibble holding the even element (R10); its scale is byte
  data_section_bytes + (o*Hkv + h)*D/16 + d/16.

The cache write [metrale: reshape_and_cache_nvfp4: each token's K and V go to
its slot_mapping slot]: slot -> (page, offset) = (slot / block_size,
slot % block_size); a negative slot is skipped (R13); bytes of slots not
written are left as they were.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .formats import (
    bf16_to_f64,
    e4m3_decode,
    e4m3_encode,
    nvfp4_encode_groups,
    nvfp4_decode_groups,
)


@dataclasses.dataclass(frozen=True)
class CacheGeometry:
    fmt: str                 # "bf16" | "fp8" | "nvfp4"
    num_pages: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    cache_stride: int = 0            # fp8: bytes per page (0 -> packed)
    block_stride_bytes: int = 0      # nvfp4: bytes per page (0 -> packed)
    data_section_bytes: int = 0      # nvfp4: code bytes at page start (0 -> packed)

    @property
    def row_elems(self) -> int:
        return self.block_size * self.num_kv_heads * self.head_dim

    def fp8_stride(self) -> int:
        return self.cache_stride or self.row_elems

    def nvfp4_sections(self):
        data = self.data_section_bytes or self.row_elems // 2
        stride = self.block_stride_bytes or data + self.row_elems // 16
        return stride, data

    def page_units(self) -> int:
        """Size of one page in the cache array's element type."""
        if self.fmt == "bf16":
            return self.row_elems
        if self.fmt == "fp8":
            return self.fp8_stride()
        return self.nvfp4_sections()[0]

    def dtype(self):
        return np.uint16 if self.fmt == "bf16" else np.uint8


def new_cache(geom: CacheGeometry, fill: int) -> np.ndarray:
    """A flat page pool of ``geom.num_pages`` pages, every unit set to ``fill``."""
    return np.full(geom.num_pages * geom.page_units(), fill, dtype=geom.dtype())


def _rows(src_bits, tokens, stride, Hkv, D):
    """Rows [n, Hkv, D] of a flat BF16 source: token t, head h at t*stride + h*D."""
    src = np.asarray(src_bits, dtype=np.uint16).reshape(-1)
    idx = tokens[:, None, None] * stride + np.arange(Hkv)[None, :, None] * D + np.arange(D)[None, None, :]
    return src[idx]


def _write_one(geom, cache, rows, page, off, scale):
    Hkv, D, bs = geom.num_kv_heads, geom.head_dim, geom.block_size
    h = np.arange(Hkv)[None, :, None]
    d = np.arange(D)[None, None, :]
    p = page[:, None, None]
    o = off[:, None, None]
    if geom.fmt == "bf16":
        cache[((p * bs + o) * Hkv + h) * D + d] = rows
    elif geom.fmt == "fp8":
        vals = bf16_to_f64(rows).astype(np.float32)
        cache[p * geom.fp8_stride() + (o * Hkv + h) * D + d] = e4m3_encode(vals, scale)
    else:
        stride, data = geom.nvfp4_sections()
        vals = bf16_to_f64(rows).astype(np.float32).reshape(rows.shape[0], Hkv, D // 16, 16)
        codes, s_codes = nvfp4_encode_groups(vals)
        codes = codes.reshape(rows.shape[0], Hkv, D)
        packed = (codes[..., 0::2] | (codes[..., 1::2] << np.uint8(4))).astype(np.uint8)
        k = np.arange(D // 2)[None, None, :]
        cache[p * stride + (o * Hkv + h) * (D // 2) + k] = packed
        g = np.arange(D // 16)[None, None, :]
        cache[p * stride + data + (o * Hkv + h) * (D // 16) + g] = s_codes


def reshape_and_cache(geom: CacheGeometry, key_bits, value_bits, k_cache, v_cache,
                      slot_mapping, key_stride=None, value_stride=None,
                      k_scale=1.0, v_scale=1.0):
    """Write every token's K and V rows (BF16 patterns, token t / head h at
    t*stride + h*head_dim) into the pools at its slot, encoding per
    ``geom.fmt``; ``k_scale``/``v_scale`` are the FP8 per-tensor scales."""
    Hkv, D, bs = geom.num_kv_heads, geom.head_dim, geom.block_size
    key_stride = Hkv * D if key_stride is None else key_stride
    value_stride = Hkv * D if value_stride is None else value_stride
    slots = np.asarray(slot_mapping, dtype=np.int64).reshape(-1)
    tokens = np.nonzero(slots >= 0)[0]
    s = slots[tokens]
    page, off = s // bs, s % bs
    _write_one(geom, k_cache, _rows(key_bits, tokens, key_stride, Hkv, D), page, off, k_scale)
    _write_one(geom, v_cache, _rows(value_bits, tokens, value_stride, Hkv, D), page, off, v_scale)


def bf16_absmax(data_bits, out_in=0.0) -> np.float32:
    """max(out_in, max_i |x_i|) over BF16 values, NaN inputs ignored (R14)
    [metrale: bf16_absmax: folded into an f32 by an atomic max, the caller
    zeroes it first]."""
    x = bf16_to_f64(np.asarray(data_bits).reshape(-1))
    x = x[~np.isnan(x)]
    m = float(np.max(np.abs(x))) if x.size else 0.0
    return np.float32(max(float(out_in), m))


def read_kv_rows(geom: CacheGeometry, cache, pages, offs, scale=1.0) -> np.ndarray:
    """Dequantized rows [n, Hkv, D] (float64, exact) at (page, offset) pairs.
    FP8 values are code * scale; NVFP4 values are E2M1 * E4M3 group scale."""
    Hkv, D, bs = geom.num_kv_heads, geom.head_dim, geom.block_size
    p = np.asarray(pages, dtype=np.int64)[:, None, None]
    o = np.asarray(offs, dtype=np.int64)[:, None, None]
    h = np.arange(Hkv)[None, :, None]
    d = np.arange(D)[None, None, :]
    if geom.fmt == "bf16":
        return bf16_to_f64(cache[((p * bs + o) * Hkv + h) * D + d])
    if geom.fmt == "fp8":
        return e4m3_decode(cache[p * geom.fp8_stride() + (o * Hkv + h) * D + d]) * float(np.float32(scale))
    stride, data = geom.nvfp4_sections()
    byte = cache[p * stride + (o * Hkv + h) * (D // 2) + d // 2]
    codes = np.where(d % 2 == 0, byte & 0xF, byte >> 4).astype(np.uint8)
    g = np.arange(D // 16)[None, None, :]
    s_codes = cache[p * stride + data + (o * Hkv + h) * (D // 16) + g]
    n = codes.shape[0]
    return nvfp4_decode_groups(codes.reshape(n, Hkv, D // 16, 16), s_codes).reshape(n, Hkv, D)
