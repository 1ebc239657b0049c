"""Python binding of the paged KV decode library (``libpkd.so``, C ABI in
``include/pkd.h``).

Argument marshalling only: torch tensors give device pointers, the current
torch stream gives the HIP stream, and every step of the computation runs in
the library's HIP kernels. There is no fallback: if the library is missing or
a call fails, a RuntimeError is raised.

Names and argument order follow the C ABI. BF16 tensors are passed as their
bit patterns (``torch.bfloat16`` storage is read as uint16 by the kernels).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "LIB_PATH", "lib", "reshape_and_cache_bf16", "reshape_and_cache_fp8",
    "reshape_and_cache_nvfp4", "bf16_absmax", "paged_decode_attn_splitk_bf16",
    "paged_decode_attn_splitk_fp8", "paged_decode_attn_splitk_nvfp4",
    "paged_decode_attn_reduce", "paged_decode_attn_splitk_append_bf16",
    "paged_decode_attn_splitk_append_fp8", "paged_decode_attn_splitk_append_nvfp4",
    "paged_decode_attn_bf16", "paged_decode_attn_fp8", "paged_decode_attn_bf16_noalloc",
    "paged_decode_attn_nvfp4", "paged_prefill_attn_bf16", "paged_prefill_attn_fp8",
    "paged_prefill_attn_nvfp4", "paged_prefill_num_splits", "contig_kv_attn_bf16",
    "contig_kv_attn_fp8", "layout_strides",
    "paged_decode_workspace_bytes", "paged_decode_num_splits",
    "pkd_status_string", "EXPORTED_SYMBOLS", "PkdError",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkd.so")

_P = ctypes.c_void_p
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64
_F32 = ctypes.c_float
_INT = ctypes.c_int

# name -> (restype, argtypes); mirrors include/pkd.h
_SIGNATURES = {
    "reshape_and_cache_bf16": (_INT, [_P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _P]),
    "reshape_and_cache_fp8": (_INT, [_P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32,
                                     _F32, _F32, _U64, _P]),
    "reshape_and_cache_nvfp4": (_INT, [_P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32,
                                       _U64, _U64, _P]),
    "bf16_absmax": (_INT, [_P, _P, _U64, _P]),
    "paged_decode_attn_splitk_bf16": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32,
                                             _F32, _U32, _U32, _U32, _U32, _P]),
    "paged_decode_attn_splitk_fp8": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32,
                                            _F32, _U32, _F32, _F32, _U32, _U64, _U32, _U32, _P]),
    "paged_decode_attn_splitk_nvfp4": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32,
                                              _F32, _U32, _U32, _U64, _U64, _U32, _U32, _P]),
    "paged_decode_attn_reduce": (_INT, [_P, _P, _P, _U32, _U32, _U32, _U32, _P]),
    "paged_decode_attn_splitk_append_bf16": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _U32, _U32,
                                                    _U32, _U32, _U32, _F32, _U32, _U32, _U32,
                                                    _U32, _U32, _U32, _P]),
    "paged_decode_attn_splitk_append_fp8": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _U32, _U32,
                                                   _U32, _U32, _U32, _F32, _U32, _F32, _F32,
                                                   _U32, _U32, _U32, _U64, _U32, _U32, _P]),
    "paged_decode_attn_splitk_append_nvfp4": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _U32, _U32,
                                                     _U32, _U32, _U32, _F32, _U32, _U32, _U32,
                                                     _U32, _U64, _U64, _U32, _U32, _P]),
    "paged_decode_attn_bf16": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32,
                                      _F32, _U32, _U32, _P, _U32, _P]),
    "paged_decode_attn_fp8": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32,
                                     _F32, _F32, _F32, _U32, _U64, _U32, _P, _U32, _P]),
    "paged_decode_attn_nvfp4": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32,
                                       _F32, _U32, _U64, _U64, _U32, _P, _U32, _P]),
    "paged_decode_attn_bf16_noalloc": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32,
                                              _U32, _F32, _U32, _U32, _U32, _P]),
    "paged_prefill_attn_bf16": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32,
                                       _U32, _U32, _F32, _U32, _U32, _U32, _U32, _P, _U32, _P]),
    "paged_prefill_attn_fp8": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32,
                                      _U32, _F32, _F32, _F32, _U32, _U32, _U64, _U32, _U32, _P,
                                      _U32, _P]),
    "paged_prefill_attn_nvfp4": (_INT, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32,
                                        _U32, _U32, _F32, _U32, _U32, _U64, _U64, _U32, _U32, _P,
                                        _U32, _P]),
    "contig_kv_attn_bf16": (_INT, [_P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _F32,
                                   _P, _U32, _U32, _P, _U32, _P]),
    "contig_kv_attn_fp8": (_INT, [_P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _F32,
                                  _F32, _F32, _P, _U32, _U32, _P, _U32, _P]),
    "paged_prefill_num_splits": (_U32, [_U32, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _U32]),
    "paged_decode_workspace_bytes": (ctypes.c_size_t, [_U32, _U32, _U32, _U32]),
    "paged_decode_num_splits": (_U32, [_U32, _U32, _U32, _U32, _U32, _U32, _U32]),
    "pkd_status_string": (ctypes.c_char_p, [_INT]),
}
EXPORTED_SYMBOLS = tuple(sorted(_SIGNATURES))

_lib = None


class PkdError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PkdError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m paged_kv_decode_splitk_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def pkd_status_string(status: int) -> str:
    return lib().pkd_status_string(int(status)).decode()


def _check(status: int, name: str):
    if status != 0:
        raise PkdError(f"{name} failed: {pkd_status_string(status)} ({status})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor, stream) -> Optional[int]:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(t.device).cuda_stream


def _num_cus(t: torch.Tensor) -> int:
    return torch.cuda.get_device_properties(t.device).multi_processor_count


def _splits_and_workspace(name, num_splits, workspace, heuristic, rows, head_dim, q):
    """num_splits None: the library's split heuristic for the device; a
    workspace must then be given whenever it picks more than one split."""
    if num_splits is None:
        num_splits = heuristic()
    if num_splits > 1 and workspace is None:
        need = paged_decode_workspace_bytes(rows[0], rows[1], head_dim, num_splits)
        raise PkdError(f"{name}: num_splits={num_splits} needs a float32 workspace of {need} "
                       "bytes (paged_decode_workspace_bytes); pass workspace=, or num_splits=1 "
                       "for the non-split path")
    return num_splits


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise PkdError("device tensors expected (the library runs on the GPU only)")


# ---------------------------------------------------------------- cache writes

def reshape_and_cache_bf16(key, value, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                           block_size, key_stride=None, value_stride=None, stream=None):
    _need_gpu(key, value, k_cache, v_cache, slot_mapping)
    n = slot_mapping.numel()
    ks = num_kv_heads * head_dim if key_stride is None else key_stride
    vs = num_kv_heads * head_dim if value_stride is None else value_stride
    _check(lib().reshape_and_cache_bf16(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(slot_mapping), n, num_kv_heads, head_dim, block_size,
                                        ks, vs, _stream(key, stream)), "reshape_and_cache_bf16")


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                          block_size, k_scale, v_scale, cache_stride=None, key_stride=None,
                          value_stride=None, stream=None):
    _need_gpu(key, value, k_cache, v_cache, slot_mapping)
    n = slot_mapping.numel()
    ks = num_kv_heads * head_dim if key_stride is None else key_stride
    vs = num_kv_heads * head_dim if value_stride is None else value_stride
    cs = block_size * num_kv_heads * head_dim if cache_stride is None else cache_stride
    _check(lib().reshape_and_cache_fp8(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(slot_mapping), n, num_kv_heads, head_dim, block_size,
                                       ks, vs, float(k_scale), float(v_scale), cs,
                                       _stream(key, stream)), "reshape_and_cache_fp8")


def nvfp4_default_sections(num_kv_heads, head_dim, block_size):
    """(block_stride_bytes, data_section_bytes) of a packed NVFP4 page."""
    data = block_size * num_kv_heads * head_dim // 2
    return data + block_size * num_kv_heads * head_dim // 16, data


def reshape_and_cache_nvfp4(key, value, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                            block_size, block_stride_bytes=None, data_section_bytes=None,
                            key_stride=None, value_stride=None, stream=None):
    _need_gpu(key, value, k_cache, v_cache, slot_mapping)
    n = slot_mapping.numel()
    ks = num_kv_heads * head_dim if key_stride is None else key_stride
    vs = num_kv_heads * head_dim if value_stride is None else value_stride
    dstride, ddata = nvfp4_default_sections(num_kv_heads, head_dim, block_size)
    bsb = dstride if block_stride_bytes is None else block_stride_bytes
    dsb = ddata if data_section_bytes is None else data_section_bytes
    _check(lib().reshape_and_cache_nvfp4(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(slot_mapping), n, num_kv_heads, head_dim,
                                         block_size, ks, vs, bsb, dsb, _stream(key, stream)),
           "reshape_and_cache_nvfp4")


def bf16_absmax(data, out_max, n_elems=None, stream=None):
    _need_gpu(data, out_max)
    n = data.numel() if n_elems is None else n_elems
    _check(lib().bf16_absmax(_ptr(data), _ptr(out_max), n, _stream(data, stream)), "bf16_absmax")


# ---------------------------------------------------------------- decode

def paged_decode_attn_splitk_bf16(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                                  max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim,
                                  block_size, scale, num_splits, q_stride, num_seqs,
                                  sliding_window=0, stream=None):
    _need_gpu(q, k_cache, v_cache, workspace, block_tables, seq_lens)
    _check(lib().paged_decode_attn_splitk_bf16(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(workspace), _ptr(block_tables),
        _ptr(seq_lens), max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), num_splits, q_stride, num_seqs, sliding_window, _stream(q, stream)),
        "paged_decode_attn_splitk_bf16")


def paged_decode_attn_splitk_fp8(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                                 max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim,
                                 block_size, scale, num_splits, k_scale, v_scale, q_stride,
                                 cache_stride, num_seqs, sliding_window=0, stream=None):
    _need_gpu(q, k_cache, v_cache, workspace, block_tables, seq_lens)
    _check(lib().paged_decode_attn_splitk_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(workspace), _ptr(block_tables),
        _ptr(seq_lens), max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), num_splits, float(k_scale), float(v_scale), q_stride, cache_stride,
        num_seqs, sliding_window, _stream(q, stream)), "paged_decode_attn_splitk_fp8")


def paged_decode_attn_splitk_nvfp4(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                                   max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim,
                                   block_size, scale, num_splits, q_stride, block_stride_bytes,
                                   data_section_bytes, num_seqs, sliding_window=0, stream=None):
    _need_gpu(q, k_cache, v_cache, workspace, block_tables, seq_lens)
    _check(lib().paged_decode_attn_splitk_nvfp4(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(workspace), _ptr(block_tables),
        _ptr(seq_lens), max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), num_splits, q_stride, block_stride_bytes, data_section_bytes, num_seqs,
        sliding_window, _stream(q, stream)), "paged_decode_attn_splitk_nvfp4")


def paged_decode_attn_reduce(workspace, output, seq_lens, num_q_heads, head_dim, num_splits,
                             num_seqs, stream=None):
    _need_gpu(workspace, output, seq_lens)
    _check(lib().paged_decode_attn_reduce(_ptr(workspace), _ptr(output), _ptr(seq_lens),
                                          num_q_heads, head_dim, num_splits, num_seqs,
                                          _stream(workspace, stream)), "paged_decode_attn_reduce")


def paged_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits) -> int:
    return int(lib().paged_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits))


def paged_decode_num_splits(num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq, block_size,
                            sliding_window=0, num_cus=256) -> int:
    return int(lib().paged_decode_num_splits(num_seqs, num_q_heads, num_kv_heads,
                                             max_blocks_per_seq, block_size, sliding_window,
                                             num_cus))


# ---------------------------------------------------------------- whole decode

def _decode_splits(name, num_splits, workspace, q, num_seqs, num_q_heads, num_kv_heads,
                   max_blocks_per_seq, block_size, sliding_window, head_dim):
    return _splits_and_workspace(
        name, num_splits, workspace,
        lambda: paged_decode_num_splits(num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq,
                                        block_size, sliding_window, _num_cus(q)),
        (num_seqs, num_q_heads), head_dim, q)


# num_splits None (the default) takes the library's split heuristic for the
# device, with the split-K pass and the combine (a workspace is then needed);
# num_splits 1 is the non-split path: one workgroup per (sequence, kv head)
# row, slow for long contexts (few rows, long serial scans).

def paged_decode_attn_bf16(q, k_cache, v_cache, output, block_tables, seq_lens,
                           max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           block_size, scale, q_stride, sliding_window=0, workspace=None,
                           num_splits=None, stream=None):
    _need_gpu(q, k_cache, v_cache, output, block_tables, seq_lens, workspace)
    num_splits = _decode_splits("paged_decode_attn_bf16", num_splits, workspace, q, num_seqs,
                                num_q_heads, num_kv_heads, max_blocks_per_seq, block_size,
                                sliding_window, head_dim)
    _check(lib().paged_decode_attn_bf16(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(output), _ptr(block_tables), _ptr(seq_lens),
        max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), q_stride, sliding_window, _ptr(workspace), num_splits,
        _stream(q, stream)), "paged_decode_attn_bf16")


def paged_decode_attn_fp8(q, k_cache, v_cache, output, block_tables, seq_lens,
                          max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim,
                          block_size, scale, k_scale, v_scale, q_stride, cache_stride,
                          sliding_window=0, workspace=None, num_splits=None, stream=None):
    _need_gpu(q, k_cache, v_cache, output, block_tables, seq_lens, workspace)
    num_splits = _decode_splits("paged_decode_attn_fp8", num_splits, workspace, q, num_seqs,
                                num_q_heads, num_kv_heads, max_blocks_per_seq, block_size,
                                sliding_window, head_dim)
    _check(lib().paged_decode_attn_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(output), _ptr(block_tables), _ptr(seq_lens),
        max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), float(k_scale), float(v_scale), q_stride, cache_stride, sliding_window,
        _ptr(workspace), num_splits, _stream(q, stream)), "paged_decode_attn_fp8")


def paged_decode_attn_nvfp4(q, k_cache, v_cache, output, block_tables, seq_lens,
                            max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, scale, q_stride, block_stride_bytes, data_section_bytes,
                            sliding_window=0, workspace=None, num_splits=None, stream=None):
    _need_gpu(q, k_cache, v_cache, output, block_tables, seq_lens, workspace)
    num_splits = _decode_splits("paged_decode_attn_nvfp4", num_splits, workspace, q, num_seqs,
                                num_q_heads, num_kv_heads, max_blocks_per_seq, block_size,
                                sliding_window, head_dim)
    _check(lib().paged_decode_attn_nvfp4(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(output), _ptr(block_tables), _ptr(seq_lens),
        max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), q_stride, block_stride_bytes, data_section_bytes, sliding_window,
        _ptr(workspace), num_splits, _stream(q, stream)),
        "paged_decode_attn_nvfp4")


SCRATCH_BYTES = 16 << 20        # PKD_SCRATCH_BYTES


def paged_decode_attn_bf16_noalloc(q, k_cache, v_cache, output, block_tables, seq_lens,
                                   max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads,
                                   head_dim, block_size, scale, q_stride, sliding_window=0,
                                   num_splits=None, stream=None):
    """paged_decode_attn_bf16 with the library's static device scratch as
    the workspace (no allocation by the caller or the library)."""
    _need_gpu(q, k_cache, v_cache, output, block_tables, seq_lens)
    if num_splits is None:
        num_splits = paged_decode_num_splits(num_seqs, num_q_heads, num_kv_heads,
                                             max_blocks_per_seq, block_size, sliding_window,
                                             _num_cus(q))
    _check(lib().paged_decode_attn_bf16_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(output), _ptr(block_tables), _ptr(seq_lens),
        max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), q_stride, sliding_window, num_splits, _stream(q, stream)),
        "paged_decode_attn_bf16_noalloc")


# ---------------------------------------------------------------- split-K with append

def paged_decode_attn_splitk_append_bf16(q, key, value, k_cache, v_cache, workspace,
                                         block_tables, seq_lens, max_blocks_per_seq, num_q_heads,
                                         num_kv_heads, head_dim, block_size, scale, num_splits,
                                         q_stride, num_seqs, sliding_window=0, key_stride=None,
                                         value_stride=None, stream=None):
    _need_gpu(q, key, value, k_cache, v_cache, workspace, block_tables, seq_lens)
    ks = num_kv_heads * head_dim if key_stride is None else key_stride
    vs = num_kv_heads * head_dim if value_stride is None else value_stride
    _check(lib().paged_decode_attn_splitk_append_bf16(
        _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(workspace),
        _ptr(block_tables), _ptr(seq_lens), max_blocks_per_seq, num_q_heads, num_kv_heads,
        head_dim, block_size, float(scale), num_splits, q_stride, ks, vs, num_seqs,
        sliding_window, _stream(q, stream)), "paged_decode_attn_splitk_append_bf16")


def paged_decode_attn_splitk_append_fp8(q, key, value, k_cache, v_cache, workspace, block_tables,
                                        seq_lens, max_blocks_per_seq, num_q_heads, num_kv_heads,
                                        head_dim, block_size, scale, num_splits, k_scale, v_scale,
                                        q_stride, cache_stride, num_seqs, sliding_window=0,
                                        key_stride=None, value_stride=None, stream=None):
    _need_gpu(q, key, value, k_cache, v_cache, workspace, block_tables, seq_lens)
    ks = num_kv_heads * head_dim if key_stride is None else key_stride
    vs = num_kv_heads * head_dim if value_stride is None else value_stride
    _check(lib().paged_decode_attn_splitk_append_fp8(
        _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(workspace),
        _ptr(block_tables), _ptr(seq_lens), max_blocks_per_seq, num_q_heads, num_kv_heads,
        head_dim, block_size, float(scale), num_splits, float(k_scale), float(v_scale), q_stride,
        ks, vs, cache_stride, num_seqs, sliding_window, _stream(q, stream)),
        "paged_decode_attn_splitk_append_fp8")


def paged_decode_attn_splitk_append_nvfp4(q, key, value, k_cache, v_cache, workspace,
                                          block_tables, seq_lens, max_blocks_per_seq,
                                          num_q_heads, num_kv_heads, head_dim, block_size, scale,
                                          num_splits, q_stride, block_stride_bytes,
                                          data_section_bytes, num_seqs, sliding_window=0,
                                          key_stride=None, value_stride=None, stream=None):
    _need_gpu(q, key, value, k_cache, v_cache, workspace, block_tables, seq_lens)
    ks = num_kv_heads * head_dim if key_stride is None else key_stride
    vs = num_kv_heads * head_dim if value_stride is None else value_stride
    _check(lib().paged_decode_attn_splitk_append_nvfp4(
        _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(workspace),
        _ptr(block_tables), _ptr(seq_lens), max_blocks_per_seq, num_q_heads, num_kv_heads,
        head_dim, block_size, float(scale), num_splits, q_stride, ks, vs, block_stride_bytes,
        data_section_bytes, num_seqs, sliding_window, _stream(q, stream)),
        "paged_decode_attn_splitk_append_nvfp4")


# ---------------------------------------------------------------- query blocks

def _prefill_splits(name, num_splits, workspace, q, num_seqs, q_len, num_q_heads, num_kv_heads,
                    max_blocks_per_seq, block_size, causal, sliding_window, head_dim):
    return _splits_and_workspace(
        name, num_splits, workspace,
        lambda: paged_prefill_num_splits(num_seqs, q_len, num_q_heads, num_kv_heads,
                                         max_blocks_per_seq, block_size, causal, sliding_window,
                                         _num_cus(q)),
        (num_seqs, num_q_heads * q_len), head_dim, q)


def _q_strides(num_q_heads, head_dim, q_len, q_stride, q_token_stride):
    ts = num_q_heads * head_dim if q_token_stride is None else q_token_stride
    qs = q_len * ts if q_stride is None else q_stride
    return qs, ts


def paged_prefill_attn_bf16(q, k_cache, v_cache, output, block_tables, seq_lens,
                            max_blocks_per_seq, num_seqs, q_len, num_q_heads, num_kv_heads,
                            head_dim, block_size, scale, causal=True, sliding_window=0,
                            q_stride=None, q_token_stride=None, workspace=None, num_splits=None,
                            stream=None):
    _need_gpu(q, k_cache, v_cache, output, block_tables, seq_lens, workspace)
    qs, ts = _q_strides(num_q_heads, head_dim, q_len, q_stride, q_token_stride)
    num_splits = _prefill_splits("paged_prefill_attn_bf16", num_splits, workspace, q, num_seqs,
                                 q_len, num_q_heads, num_kv_heads, max_blocks_per_seq,
                                 block_size, causal, sliding_window, head_dim)
    _check(lib().paged_prefill_attn_bf16(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(output), _ptr(block_tables), _ptr(seq_lens),
        max_blocks_per_seq, num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), qs, ts, int(bool(causal)), sliding_window, _ptr(workspace), num_splits,
        _stream(q, stream)), "paged_prefill_attn_bf16")


def paged_prefill_attn_fp8(q, k_cache, v_cache, output, block_tables, seq_lens,
                           max_blocks_per_seq, num_seqs, q_len, num_q_heads, num_kv_heads,
                           head_dim, block_size, scale, k_scale, v_scale, cache_stride,
                           causal=True, sliding_window=0, q_stride=None, q_token_stride=None,
                           workspace=None, num_splits=None, stream=None):
    _need_gpu(q, k_cache, v_cache, output, block_tables, seq_lens, workspace)
    qs, ts = _q_strides(num_q_heads, head_dim, q_len, q_stride, q_token_stride)
    num_splits = _prefill_splits("paged_prefill_attn_fp8", num_splits, workspace, q, num_seqs,
                                 q_len, num_q_heads, num_kv_heads, max_blocks_per_seq,
                                 block_size, causal, sliding_window, head_dim)
    _check(lib().paged_prefill_attn_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(output), _ptr(block_tables), _ptr(seq_lens),
        max_blocks_per_seq, num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), float(k_scale), float(v_scale), qs, ts, cache_stride, int(bool(causal)),
        sliding_window, _ptr(workspace), num_splits, _stream(q, stream)),
        "paged_prefill_attn_fp8")


def paged_prefill_attn_nvfp4(q, k_cache, v_cache, output, block_tables, seq_lens,
                             max_blocks_per_seq, num_seqs, q_len, num_q_heads, num_kv_heads,
                             head_dim, block_size, scale, block_stride_bytes, data_section_bytes,
                             causal=True, sliding_window=0, q_stride=None, q_token_stride=None,
                             workspace=None, num_splits=None, stream=None):
    _need_gpu(q, k_cache, v_cache, output, block_tables, seq_lens, workspace)
    qs, ts = _q_strides(num_q_heads, head_dim, q_len, q_stride, q_token_stride)
    num_splits = _prefill_splits("paged_prefill_attn_nvfp4", num_splits, workspace, q, num_seqs,
                                 q_len, num_q_heads, num_kv_heads, max_blocks_per_seq,
                                 block_size, causal, sliding_window, head_dim)
    _check(lib().paged_prefill_attn_nvfp4(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(output), _ptr(block_tables), _ptr(seq_lens),
        max_blocks_per_seq, num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, block_size,
        float(scale), qs, ts, block_stride_bytes, data_section_bytes, int(bool(causal)),
        sliding_window, _ptr(workspace), num_splits, _stream(q, stream)),
        "paged_prefill_attn_nvfp4")


def paged_prefill_num_splits(num_seqs, q_len, num_q_heads, num_kv_heads, max_blocks_per_seq,
                             block_size, causal=True, sliding_window=0, num_cus=256) -> int:
    return int(lib().paged_prefill_num_splits(num_seqs, q_len, num_q_heads, num_kv_heads,
                                              max_blocks_per_seq, block_size, int(bool(causal)),
                                              sliding_window, num_cus))


# ---------------------------------------------------------------- contiguous K/V

def layout_strides(layout, num_seqs, length, num_heads, head_dim):
    """Element strides (sequence, token, head) of a dense tensor in the
    "blhd" (b, l, h, d) or "bhld" (b, h, l, d) layout."""
    if layout == "blhd":
        return (length * num_heads * head_dim, num_heads * head_dim, head_dim)
    if layout == "bhld":
        return (num_heads * length * head_dim, head_dim, length * head_dim)
    raise PkdError(f"unknown layout {layout!r} (blhd or bhld)")


def _strides_arg(q_strides, k_strides, v_strides, o_strides):
    vals = [int(x) for x in (*q_strides, *k_strides, *v_strides, *o_strides)]
    if len(vals) != 12:
        raise PkdError("three strides each for q, k, v and the output")
    return (ctypes.c_uint64 * 12)(*vals)


def contig_kv_attn_bf16(q, k, v, output, seq_lens, num_seqs, q_len, max_seq_len, num_q_heads,
                        num_kv_heads, head_dim, scale, q_strides, k_strides, v_strides,
                        o_strides, causal=True, sliding_window=0, workspace=None, num_splits=None,
                        stream=None):
    _need_gpu(q, k, v, output, seq_lens, workspace)
    st = _strides_arg(q_strides, k_strides, v_strides, o_strides)
    num_splits = _splits_and_workspace(
        "contig_kv_attn_bf16", num_splits, workspace,
        lambda: paged_prefill_num_splits(num_seqs, q_len, num_q_heads, num_kv_heads,
                                         (max_seq_len + 15) // 16, 16, causal, sliding_window,
                                         _num_cus(q)),
        (num_seqs, num_q_heads * q_len), head_dim, q)
    _check(lib().contig_kv_attn_bf16(
        _ptr(q), _ptr(k), _ptr(v), _ptr(output), _ptr(seq_lens), num_seqs, q_len, max_seq_len,
        num_q_heads, num_kv_heads, head_dim, float(scale), st, int(bool(causal)),
        sliding_window, _ptr(workspace), num_splits, _stream(q, stream)), "contig_kv_attn_bf16")


def contig_kv_attn_fp8(q, k, v, output, seq_lens, num_seqs, q_len, max_seq_len, num_q_heads,
                       num_kv_heads, head_dim, scale, k_scale, v_scale, q_strides, k_strides,
                       v_strides, o_strides, causal=True, sliding_window=0, workspace=None,
                       num_splits=None, stream=None):
    _need_gpu(q, k, v, output, seq_lens, workspace)
    st = _strides_arg(q_strides, k_strides, v_strides, o_strides)
    num_splits = _splits_and_workspace(
        "contig_kv_attn_fp8", num_splits, workspace,
        lambda: paged_prefill_num_splits(num_seqs, q_len, num_q_heads, num_kv_heads,
                                         (max_seq_len + 15) // 16, 16, causal, sliding_window,
                                         _num_cus(q)),
        (num_seqs, num_q_heads * q_len), head_dim, q)
    _check(lib().contig_kv_attn_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(output), _ptr(seq_lens), num_seqs, q_len, max_seq_len,
        num_q_heads, num_kv_heads, head_dim, float(scale), float(k_scale), float(v_scale), st,
        int(bool(causal)), sliding_window, _ptr(workspace), num_splits, _stream(q, stream)),
        "contig_kv_attn_fp8")
