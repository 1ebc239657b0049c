"""Helpers for the GPU parity tests: device pools written through the
library, oracle pools written by the oracle from the same seeded inputs, and
the comparison rule. Nothing here computes attention or encodes values."""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np
import torch

import oracle
import paged_kv_decode_splitk_amd as pkd

POISON = {"bf16": 0x7FC0, "fp8": 0x7F, "nvfp4": 0x7F}    # NaN patterns
ATOL = 1e-2
RTOL = 1e-2


def dev():
    return torch.device("cuda:0")


def u16_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(dev())


def i32_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def pool_to_np(t: torch.Tensor, fmt: str) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if fmt == "bf16" else a.view(np.uint8)


def geometry(w, fmt=None, cache_stride=0, block_stride_bytes=0, data_section_bytes=0):
    fmt = fmt or w.kv_dtype
    return oracle.CacheGeometry(fmt, w.num_pages, w.block_size, w.num_kv_heads, w.head_dim,
                                cache_stride=cache_stride, block_stride_bytes=block_stride_bytes,
                                data_section_bytes=data_section_bytes)


def alloc_pool(geom, fill) -> torch.Tensor:
    n = geom.num_pages * geom.page_units()
    if geom.fmt == "bf16":
        return torch.full((n,), np.int16(np.uint16(fill).view(np.int16)), dtype=torch.int16,
                          device=dev())
    return torch.full((n,), int(fill), dtype=torch.uint8, device=dev())


def gpu_absmax(bits: np.ndarray) -> float:
    out = torch.zeros(1, dtype=torch.float32, device=dev())
    x = u16_to_dev(bits.reshape(-1))
    pkd.bf16_absmax(x, out)
    torch.cuda.synchronize()
    return float(out.item())


class DeviceKV:
    """K/V pools on the GPU, filled by the library's cache write."""

    def __init__(self, w, geom, k_scale=1.0, v_scale=1.0, fill=None, tokens=None):
        self.w, self.geom = w, geom
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        fill = POISON[geom.fmt] if fill is None else fill
        self.k = alloc_pool(geom, fill)
        self.v = alloc_pool(geom, fill)
        sel = slice(None) if tokens is None else tokens
        key = u16_to_dev(w.k_bits[sel].reshape(-1, w.num_kv_heads * w.head_dim))
        val = u16_to_dev(w.v_bits[sel].reshape(-1, w.num_kv_heads * w.head_dim))
        slots = i32_to_dev(w.slot_mapping[sel])
        Hkv, D, bs = w.num_kv_heads, w.head_dim, w.block_size
        if geom.fmt == "bf16":
            pkd.reshape_and_cache_bf16(key, val, self.k, self.v, slots, Hkv, D, bs)
        elif geom.fmt == "fp8":
            pkd.reshape_and_cache_fp8(key, val, self.k, self.v, slots, Hkv, D, bs, k_scale,
                                      v_scale, cache_stride=geom.fp8_stride())
        else:
            stride, data = geom.nvfp4_sections()
            pkd.reshape_and_cache_nvfp4(key, val, self.k, self.v, slots, Hkv, D, bs,
                                        block_stride_bytes=stride, data_section_bytes=data)
        del key, val, slots

    def decode(self, num_splits, q_bits=None, sliding_window=None, q_stride=None, seq_lens=None,
               return_ws=False, ws_fill=None):
        w, g = self.w, self.geom
        B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
        q_bits = w.q_bits if q_bits is None else q_bits
        q_stride = Hq * D if q_stride is None else q_stride
        window = w.sliding_window if sliding_window is None else sliding_window
        lens_np = w.seq_lens if seq_lens is None else seq_lens
        q = u16_to_dev(q_bits.reshape(-1))
        bt = i32_to_dev(w.block_tables)
        lens = i32_to_dev(lens_np)
        ws = torch.empty(pkd.paged_decode_workspace_bytes(B, Hq, D, num_splits) // 4,
                         dtype=torch.float32, device=dev())
        if ws_fill is not None:
            ws.fill_(ws_fill)
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev())
        common = (q, self.k, self.v, ws, bt, lens, w.max_blocks_per_seq, Hq, Hkv, D, bs,
                  float(w.scale), num_splits)
        if g.fmt == "bf16":
            pkd.paged_decode_attn_splitk_bf16(*common, q_stride, B, window)
        elif g.fmt == "fp8":
            pkd.paged_decode_attn_splitk_fp8(*common, self.k_scale, self.v_scale, q_stride,
                                             g.fp8_stride(), B, window)
        else:
            stride, data = g.nvfp4_sections()
            pkd.paged_decode_attn_splitk_nvfp4(*common, q_stride, stride, data, B, window)
        pkd.paged_decode_attn_reduce(ws, out, lens, Hq, D, num_splits, B)
        torch.cuda.synchronize()
        res = out.float().cpu().numpy().astype(np.float64)
        if return_ws:
            return res, ws.cpu().numpy().reshape(B, Hq, num_splits, D + 2)
        return res


    def decode_single(self, num_splits, q_bits=None, out=None):
        """The whole-decode call (one wave per row when num_splits is 1)."""
        w, g = self.w, self.geom
        B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
        q_bits = w.q_bits if q_bits is None else q_bits
        q = u16_to_dev(q_bits.reshape(-1))
        bt = i32_to_dev(w.block_tables)
        lens = i32_to_dev(w.seq_lens)
        ws = None
        if num_splits > 1:
            ws = torch.full((pkd.paged_decode_workspace_bytes(B, Hq, D, num_splits) // 4,),
                            float("nan"), dtype=torch.float32, device=dev())
        if out is None:
            out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=dev())
        common = (q, self.k, self.v, out, bt, lens, w.max_blocks_per_seq, B, Hq, Hkv, D, bs,
                  float(w.scale))
        tail = dict(sliding_window=w.sliding_window, workspace=ws, num_splits=num_splits)
        if g.fmt == "bf16":
            pkd.paged_decode_attn_bf16(*common, Hq * D, **tail)
        elif g.fmt == "fp8":
            pkd.paged_decode_attn_fp8(*common, self.k_scale, self.v_scale, Hq * D,
                                      g.fp8_stride(), **tail)
        else:
            stride, data = g.nvfp4_sections()
            pkd.paged_decode_attn_nvfp4(*common, Hq * D, stride, data, **tail)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)


    def prefill(self, q_bits, q_len, num_splits, causal=True, sliding_window=None,
                q_stride=None, q_token_stride=None, return_ws=False, ws_fill=float("nan")):
        """The multi-token call: q_bits holds q_len tokens per sequence."""
        w, g = self.w, self.geom
        B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
        window = w.sliding_window if sliding_window is None else sliding_window
        q = u16_to_dev(np.asarray(q_bits).reshape(-1))
        bt = i32_to_dev(w.block_tables)
        lens = i32_to_dev(w.seq_lens)
        ws = None
        if num_splits > 1:
            ws = torch.full((pkd.paged_decode_workspace_bytes(B, Hq * q_len, D, num_splits) // 4,),
                            ws_fill, dtype=torch.float32, device=dev())
        out = torch.full((B, q_len, Hq, D), float("nan"), dtype=torch.bfloat16, device=dev())
        common = (q, self.k, self.v, out, bt, lens, w.max_blocks_per_seq, B, q_len, Hq, Hkv, D,
                  bs, float(w.scale))
        tail = dict(causal=causal, sliding_window=window, q_stride=q_stride,
                    q_token_stride=q_token_stride, workspace=ws, num_splits=num_splits)
        if g.fmt == "bf16":
            pkd.paged_prefill_attn_bf16(*common, **tail)
        elif g.fmt == "fp8":
            pkd.paged_prefill_attn_fp8(*common, self.k_scale, self.v_scale, g.fp8_stride(), **tail)
        else:
            stride, data = g.nvfp4_sections()
            pkd.paged_prefill_attn_nvfp4(*common, stride, data, **tail)
        torch.cuda.synchronize()
        res = out.float().cpu().numpy().astype(np.float64)
        if return_ws:
            return res, ws.cpu().numpy().reshape(B, q_len, Hq, num_splits, D + 2)
        return res


ORACLE_CHUNK = 4096          # tokens per oracle cache-write call
ORACLE_THREADS = min(16, len(os.sched_getaffinity(0)))


def oracle_pools(w, geom, k_scale=1.0, v_scale=1.0, seqs=None, fill=None):
    """Oracle pools written by the oracle's cache write (all tokens, or only
    the tokens of the sequences in ``seqs``). The tokens go through the
    oracle in chunks on a few host threads: slots are unique, so the chunks
    write disjoint bytes, and small chunks keep the encoders' float64
    temporaries small."""
    fill = POISON[geom.fmt] if fill is None else fill
    kc, vc = oracle.new_cache(geom, fill), oracle.new_cache(geom, fill)
    if seqs is None:
        tok = np.arange(w.num_tokens)
    else:
        tok = np.nonzero(np.isin(w.token_seq, np.asarray(seqs)))[0]

    def write(part):
        oracle.reshape_and_cache(geom, w.k_bits[part], w.v_bits[part], kc, vc,
                                 w.slot_mapping[part], k_scale=k_scale, v_scale=v_scale)

    parts = [tok[i:i + ORACLE_CHUNK] for i in range(0, tok.size, ORACLE_CHUNK)]
    if len(parts) <= 1:
        for part in parts:
            write(part)
    else:
        with concurrent.futures.ThreadPoolExecutor(ORACLE_THREADS) as ex:
            list(ex.map(write, parts))
    return kc, vc


def oracle_decode(w, geom, kc, vc, k_scale=1.0, v_scale=1.0, seqs=None, q_bits=None,
                  sliding_window=None, q_stride=None, seq_lens=None):
    return oracle.paged_decode_attention(
        geom, w.q_bits if q_bits is None else q_bits, kc, vc, w.block_tables,
        w.seq_lens if seq_lens is None else seq_lens, w.num_q_heads, w.scale, q_stride=q_stride,
        sliding_window=w.sliding_window if sliding_window is None else sliding_window,
        k_scale=k_scale, v_scale=v_scale, seqs=seqs)


def assert_close(got, ref, what=""):
    err = np.abs(got - ref)
    bad = ~(err <= ATOL + RTOL * np.abs(ref))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside atol=rtol=1e-2; "
                             f"max err {np.nanmax(err):.3e}; first {idx.tolist()}")
    return float(err.max()) if err.size else 0.0


_FULL = {}


def full_size_reference(name):
    """(workload, geometry, k_scale, v_scale, oracle K pool, oracle V pool,
    oracle decode of every sequence) of a full-size workload, built once per
    test session: every token goes through the oracle's cache write and
    every sequence through its decode."""
    if name not in _FULL:
        import workloads
        w = workloads.make_workload(name)
        geom = geometry(w)
        ks, vs = fp8_scales(w) if w.kv_dtype == "fp8" else (1.0, 1.0)
        kc, vc = oracle_pools(w, geom, ks, vs)
        ref = oracle_decode(w, geom, kc, vc, ks, vs)
        _FULL[name] = (w, geom, ks, vs, kc, vc, ref)
    return _FULL[name]


def fp8_scales(w):
    """Per-tensor FP8 scales from the GPU absmax (K, then V) and from the
    oracle's absmax; they must agree bit for bit."""
    k_gpu = gpu_absmax(w.k_bits)
    v_gpu = gpu_absmax(w.v_bits)
    k_ref = np.float32(0.0)
    v_ref = np.float32(0.0)
    flat_k = w.k_bits.reshape(-1)
    flat_v = w.v_bits.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_k.size, step):
        k_ref = oracle.bf16_absmax(flat_k[i:i + step], k_ref)
        v_ref = oracle.bf16_absmax(flat_v[i:i + step], v_ref)
    assert np.float32(k_gpu) == k_ref and np.float32(v_gpu) == v_ref
    return np.float32(k_ref) / np.float32(448.0), np.float32(v_ref) / np.float32(448.0)


def oracle_prefill(w, geom, kc, vc, q_bits, q_len, causal=True, k_scale=1.0, v_scale=1.0,
                   seqs=None, sliding_window=None, return_state=False):
    return oracle.paged_prefill_attention(
        geom, q_bits, kc, vc, w.block_tables, w.seq_lens, w.num_q_heads, q_len, w.scale,
        causal=causal, sliding_window=w.sliding_window if sliding_window is None else sliding_window,
        k_scale=k_scale, v_scale=v_scale, seqs=seqs, return_state=return_state)


# ------------------------------------------------------------------ contiguous K/V

def _tensor(rows, layout, Lmax, fill, dtype):
    """Per-sequence rows [L, Hkv, D] laid into (b, l, h, d) or (b, h, l, d)."""
    B = len(rows)
    Hkv, D = rows[0].shape[1], rows[0].shape[2]
    t = np.full((B, Lmax, Hkv, D), fill, dtype)
    for b, r in enumerate(rows):
        t[b, :len(r)] = r
    if layout == "bhld":
        t = np.ascontiguousarray(t.transpose(0, 2, 1, 3))
    return t, pkd.layout_strides(layout, B, Lmax, Hkv, D)


def _seq_rows(w, bits):
    out, start = [], 0
    for L in w.seq_lens:
        out.append(bits[start:start + int(L)])
        start += int(L)
    return out


class Contig:
    """A workload's K/V as contiguous device tensors (BF16, or FP8 codes from
    the oracle's encoder: inputs, read the same by both sides)."""

    def __init__(self, w, layout, fmt="bf16", k_scale=1.0, v_scale=1.0, pad=3, Lmax=None):
        self.w, self.fmt = w, fmt
        self.Lmax = int(max(1, w.seq_lens.max(initial=1))) + pad if Lmax is None else Lmax
        kr, vr = _seq_rows(w, w.k_bits), _seq_rows(w, w.v_bits)
        if fmt == "fp8":
            kr = [oracle.e4m3_encode(oracle.bf16_to_f64(r).astype(np.float32), k_scale) for r in kr]
            vr = [oracle.e4m3_encode(oracle.bf16_to_f64(r).astype(np.float32), v_scale) for r in vr]
            fill, dt = 0x7F, np.uint8                          # NaN codes in the padding
        else:
            fill, dt = 0x7FC0, np.uint16
        self.k_np, self.ks = _tensor(kr, layout, self.Lmax, fill, dt)
        self.v_np, self.vs = _tensor(vr, layout, self.Lmax, fill, dt)
        if fmt == "fp8":
            self.k = torch.from_numpy(self.k_np.reshape(-1)).to(dev())
            self.v = torch.from_numpy(self.v_np.reshape(-1)).to(dev())
        else:
            self.k = u16_to_dev(self.k_np.reshape(-1))
            self.v = u16_to_dev(self.v_np.reshape(-1))
        self.k_scale, self.v_scale = k_scale, v_scale

    def run(self, q, q_len, num_splits, causal=True, window=None, q_strides=None,
            o_layout="blhd", o_pad=0):
        w = self.w
        B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
        window = w.sliding_window if window is None else window
        if q_strides is None:
            q_strides = (q_len * Hq * D, Hq * D, D)
        # output: (b, i, h, d) or (b, h, i, d), each head row padded by o_pad elements
        row = D + o_pad
        if o_layout == "blhd":
            os_ = (q_len * Hq * row, Hq * row, row)
        else:
            os_ = (Hq * q_len * row, row, q_len * row)
        out = torch.full((B * q_len * Hq * row,), float("nan"), dtype=torch.bfloat16, device=dev())
        ws = None
        if num_splits > 1:
            ws = torch.full((pkd.paged_decode_workspace_bytes(B, Hq * q_len, D, num_splits) // 4,),
                            float("nan"), dtype=torch.float32, device=dev())
        qd = u16_to_dev(np.asarray(q).reshape(-1))
        lens = i32_to_dev(w.seq_lens)
        args = (qd, self.k, self.v, out, lens, B, q_len, self.Lmax, Hq, Hkv, D, float(w.scale))
        kw = dict(causal=causal, sliding_window=window, workspace=ws, num_splits=num_splits)
        if self.fmt == "fp8":
            pkd.contig_kv_attn_fp8(*args, self.k_scale, self.v_scale, q_strides, self.ks, self.vs,
                                   os_, **kw)
        else:
            pkd.contig_kv_attn_bf16(*args, q_strides, self.ks, self.vs, os_, **kw)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy().astype(np.float64)
        idx = (np.arange(B)[:, None, None, None] * os_[0] + np.arange(q_len)[None, :, None, None] * os_[1]
               + np.arange(Hq)[None, None, :, None] * os_[2] + np.arange(D)[None, None, None, :])
        return o[idx]

    def oracle(self, q, q_len, causal=True, window=None, q_strides=None, seqs=None):
        w = self.w
        Hq, D = w.num_q_heads, w.head_dim
        if q_strides is None:
            q_strides = (q_len * Hq * D, Hq * D, D)
        return oracle.contiguous_attention(
            self.fmt, q, self.k_np, self.v_np, w.seq_lens, Hq, w.num_kv_heads, D, q_len, w.scale,
            q_strides, self.ks, self.vs, causal=causal,
            sliding_window=w.sliding_window if window is None else window,
            k_scale=self.k_scale, v_scale=self.v_scale, seqs=seqs)
