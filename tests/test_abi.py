"""The C ABI library on the CPU (no GPU calls): it loads, exports exactly the
symbols include/pkd.h declares, its host helpers compute what the header
states, and argument validation returns the documented status codes before
anything is launched."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import paged_kv_decode_splitk_amd as pkd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkd.h")


def _header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"PKD_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkd.LIB_PATH):
        pytest.skip("libpkd.so not built")
    return pkd.lib()


def test_header_and_binding_agree():
    assert _header_symbols() == list(pkd.EXPORTED_SYMBOLS)


def test_library_exports_exactly_the_header_symbols(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pkd.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    text_syms = sorted(line.split()[-1] for line in out.splitlines()
                       if len(line.split()) == 3 and line.split()[1] in ("T", "t"))
    assert text_syms == _header_symbols()


def test_workspace_bytes(lib):
    assert pkd.paged_decode_workspace_bytes(32, 32, 128, 8) == 32 * 32 * 8 * 130 * 4
    assert pkd.paged_decode_workspace_bytes(1, 1, 64, 1) == 66 * 4
    assert pkd.paged_decode_workspace_bytes(0, 32, 128, 8) == 0


def test_num_splits_heuristic(lib):
    ns = pkd.paged_decode_num_splits
    # 1 + 4 * (4 waves per CU * CUs) / rows, at most one piece per 16-key tile
    assert ns(1, 32, 8, 2048, 16, 0, 256) == 513          # B=1, 32K keys: 8 rows
    assert ns(32, 32, 8, 256, 16, 0, 256) == 17           # B=32: 256 rows
    assert ns(1, 32, 8, 64, 16, 0, 256) == 64             # B=1, 1K keys: capped by 64 tiles
    assert ns(2, 4, 2, 4, 16, 0, 256) == 4
    assert ns(64, 16, 8, 512, 16, 4096, 256) == 9         # 512 rows
    assert ns(1, 16, 8, 512, 16, 4096, 256) == 257        # window: 257 tiles at most
    assert ns(1, 64, 1, 4096, 16, 0, 256) == 1025         # 4 rows (16-q-head chunks)
    assert ns(4096, 8, 8, 10, 16, 0, 256) == 2
    assert ns(3, 8, 8, 1, 16, 0, 0) == 1                  # a single tile per row
    assert ns(0, 8, 8, 10, 16, 0, 256) == 1


def test_status_strings(lib):
    assert pkd.pkd_status_string(0) == "ok"
    assert pkd.pkd_status_string(-1) == "invalid argument"
    assert pkd.pkd_status_string(-2) == "unsupported shape"
    assert pkd.pkd_status_string(-3) == "kernel launch failed"
    assert pkd.pkd_status_string(-4) == "workspace larger than the static scratch"
    assert pkd.pkd_status_string(7) == "unknown status"


A16 = 0x10000          # a 16-byte aligned, never dereferenced address


def _decode(lib, **kw):
    args = dict(q=A16, kc=A16, vc=A16, ws=A16, bt=A16, lens=A16, maxb=4, Hq=4, Hkv=2, D=64,
                bs=16, scale=0.125, S=1, q_stride=256, B=2, W=0)
    args.update(kw)
    a = args
    return lib.paged_decode_attn_splitk_bf16(a["q"], a["kc"], a["vc"], a["ws"], a["bt"], a["lens"],
                                             a["maxb"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                                             a["scale"], a["S"], a["q_stride"], a["B"], a["W"],
                                             None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1),
    (dict(ws=None), -1),
    (dict(q=A16 + 2), -1),              # misaligned
    (dict(Hq=5), -1),                   # not a multiple of the kv heads
    (dict(Hkv=0), -1),
    (dict(maxb=0), -1),
    (dict(q_stride=200), -1),           # shorter than Hq * D
    (dict(q_stride=260), -1),           # not a multiple of 8
    (dict(D=96), -2),
    (dict(D=1024), -2),
    (dict(bs=8), -2),
    (dict(bs=48), -2),
    (dict(S=0), -2),
    (dict(S=4097), -2),
    # more than 2^30 16-key tiles in one launch: 2^16 sequences x 4 kv heads x
    # 2^13 pages (rejected before anything is launched or read)
    (dict(B=1 << 16, Hq=4, Hkv=4, maxb=1 << 13, q_stride=256, S=2), -2),
])
def test_decode_validation(lib, kw, status):
    assert _decode(lib, **kw) == status


def test_zero_work_calls_are_noops(lib):
    assert _decode(lib, B=0, q=None, ws=None) == 0
    assert lib.reshape_and_cache_bf16(None, None, None, None, None, 0, 2, 64, 16, 128, 128, None) == 0
    assert lib.bf16_absmax(None, None, 0, None) == 0
    assert lib.paged_decode_attn_reduce(None, None, None, 4, 64, 1, 0, None) == 0


def test_fp8_nvfp4_specific_validation(lib):
    f8 = lib.paged_decode_attn_splitk_fp8
    ok = (A16, A16, A16, A16, A16, A16, 4, 4, 2, 64, 16, 0.125, 1, 1.0, 1.0, 256)
    assert f8(*ok, 16 * 2 * 64 - 16, 2, 0, None) == -1     # cache stride shorter than a page
    assert f8(*ok, 16 * 2 * 64 + 8, 2, 0, None) == -1      # not a multiple of 16
    n4 = lib.paged_decode_attn_splitk_nvfp4
    ok4 = (A16, A16, A16, A16, A16, A16, 4, 4, 2, 64, 16, 0.125, 1, 256)
    data = 16 * 2 * 64 // 2
    assert n4(*ok4, data + 128, data - 16, 2, 0, None) == -1   # data section too small
    assert n4(*ok4, data + 64, data, 2, 0, None) == -1         # no room for the scales
    assert n4(*ok4, data + 128 + 8, data, 2, 0, None) == -1    # stride not a multiple of 16
    w = lib.reshape_and_cache_nvfp4
    assert w(A16, A16, A16, A16, A16, 3, 2, 64, 16, 128, 128, data + 64, data, None) == -1
    wf = lib.reshape_and_cache_fp8
    assert wf(A16, A16, A16, A16, A16, 3, 2, 64, 16, 120, 128, 1.0, 1.0, 2048, None) == -1
    assert wf(A16, A16, A16, A16, A16, 3, 2, 64, 16, 132, 128, 1.0, 1.0, 2048, None) == -1
    assert lib.bf16_absmax(A16 + 2, A16, 10, None) == -1
    assert lib.paged_decode_attn_reduce(A16, A16, A16, 4, 96, 1, 2, None) == -2
    assert lib.paged_decode_attn_reduce(A16, A16, None, 4, 64, 1, 2, None) == -1


def test_whole_decode_validation(lib):
    f = lib.paged_decode_attn_bf16
    # q, k, v, out, bt, lens, maxb, B, Hq, Hkv, D, bs, scale, q_stride, W, ws, S
    base = [A16, A16, A16, A16, A16, A16, 4, 2, 4, 2, 64, 16, 0.125, 256, 0, A16, 2, None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[{"out": 3, "ws": 15, "S": 16, "Hq": 8, "D": 10, "q": 0}[k]] = v
        return f(*a)

    assert call(out=None) == -1                 # the output is always needed
    assert call(out=A16 + 8) == -1              # 16-byte aligned
    assert call(ws=None) == -1                  # num_splits > 1: workspace needed
    assert call(S=0) == -2
    assert call(S=4097) == -2
    assert call(Hq=5) == -1
    assert call(D=96) == -2
    assert call(q=None) == -1
    assert f(None, None, None, None, None, None, 4, 0, 4, 2, 64, 16, 0.125, 256, 0, None, 1,
             None) == 0                         # no sequences: a no-op
    f8 = lib.paged_decode_attn_fp8
    assert f8(A16, A16, A16, A16, A16, A16, 4, 2, 4, 2, 64, 16, 0.125, 1.0, 1.0, 256,
              16 * 2 * 64 - 16, 0, A16, 2, None) == -1               # cache stride too short
    n4 = lib.paged_decode_attn_nvfp4
    data = 16 * 2 * 64 // 2
    assert n4(A16, A16, A16, A16, A16, A16, 4, 2, 4, 2, 64, 16, 0.125, 256, data + 64, data, 0,
              A16, 2, None) == -1                                      # no room for the scales


def test_append_validation(lib):
    f = lib.paged_decode_attn_splitk_append_bf16
    # q, key, value, kc, vc, ws, bt, lens, maxb, Hq, Hkv, D, bs, scale, S, q_stride, ks, vs, B, W
    base = [A16, A16, A16, A16, A16, A16, A16, A16, 4, 4, 2, 64, 16, 0.125, 2, 256, 128, 128, 2, 0,
            None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[{"key": 1, "value": 2, "ks": 16, "vs": 17, "B": 18, "D": 11}[k]] = v
        return f(*a)

    assert call(key=None) == -1
    assert call(value=A16 + 4) == -1            # 16-byte aligned
    assert call(ks=120) == -1                   # shorter than num_kv_heads * head_dim
    assert call(vs=132) == -1                   # not a multiple of 8
    assert call(D=96) == -2
    assert call(B=0, key=None) == 0             # no sequences: a no-op
    f8 = lib.paged_decode_attn_splitk_append_fp8
    assert f8(A16, None, A16, A16, A16, A16, A16, A16, 4, 4, 2, 64, 16, 0.125, 2, 1.0, 1.0, 256,
              128, 128, 2048, 2, 0, None) == -1
    n4 = lib.paged_decode_attn_splitk_append_nvfp4
    data = 16 * 2 * 64 // 2
    assert n4(A16, A16, A16, A16, A16, A16, A16, A16, 4, 4, 2, 64, 16, 0.125, 2, 256, 128, 128,
              data + 64, data, 2, 0, None) == -1                    # no room for the scales


def test_prefill_validation(lib):
    f = lib.paged_prefill_attn_bf16
    # q, k, v, out, bt, lens, maxb, B, q_len, Hq, Hkv, D, bs, scale, q_stride, tok_stride,
    # causal, W, ws, S
    base = [A16, A16, A16, A16, A16, A16, 4, 2, 3, 4, 2, 64, 16, 0.125, 3 * 256, 256, 1, 0, A16,
            2, None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[{"out": 3, "B": 7, "n": 8, "Hq": 9, "D": 11, "qs": 14, "ts": 15, "ws": 18,
               "S": 19}[k]] = v
        return f(*a)

    assert call(n=0) == -1                      # no query tokens
    assert call(n=4097, qs=4097 * 256) == -2    # longer than the supported block
    assert call(ts=248) == -1                   # token rows overlap
    assert call(ts=260) == -1                   # not a multiple of 8
    assert call(qs=3 * 256 - 8) == -1           # the last token runs past the sequence stride
    assert call(out=None) == -1
    assert call(ws=None) == -1                  # num_splits > 1: workspace needed
    assert call(D=96) == -2
    assert call(Hq=5) == -1
    assert call(B=0, out=None) == 0             # no sequences: a no-op
    f8 = lib.paged_prefill_attn_fp8
    assert f8(A16, A16, A16, A16, A16, A16, 4, 2, 3, 4, 2, 64, 16, 0.125, 1.0, 1.0, 768, 256,
              16 * 2 * 64 - 16, 1, 0, A16, 2, None) == -1           # cache stride too short
    n4 = lib.paged_prefill_attn_nvfp4
    data = 16 * 2 * 64 // 2
    assert n4(A16, A16, A16, A16, A16, A16, 4, 2, 3, 4, 2, 64, 16, 0.125, 768, 256, data + 64,
              data, 1, 0, A16, 2, None) == -1                       # no room for the scales


def test_prefill_num_splits(lib):
    ns = lib.paged_prefill_num_splits
    dec = lib.paged_decode_num_splits
    # q_len tokens of G heads count as q_len * G query heads
    assert ns(32, 4, 32, 8, 256, 16, 1, 0, 256) == dec(32, 128, 8, 256, 16, 0, 256)
    assert ns(1, 1, 32, 8, 2048, 16, 1, 0, 256) == dec(1, 32, 8, 2048, 16, 0, 256)
    # a causal window widens by q_len - 1 keys; a plain one does not
    assert ns(1, 8, 32, 8, 2048, 16, 1, 64, 256) == dec(1, 256, 8, 2048, 16, 71, 256)
    assert ns(1, 8, 32, 8, 2048, 16, 0, 64, 256) == dec(1, 256, 8, 2048, 16, 64, 256)
    assert ns(1, 0, 32, 8, 2048, 16, 1, 0, 256) == 1
    # wider than 32 columns: rows of 128 columns (waves sharing each tile), so
    # 32 sequences x 8 kv heads x 1 row want 1 + 4096 / 256 = 17 pieces a row
    assert ns(32, 16, 32, 8, 256, 16, 1, 0, 256) == 17
    assert ns(32, 64, 32, 8, 256, 16, 1, 0, 256) == 1 + -(-4096 // 512)


def test_contig_validation(lib):
    import ctypes
    f = lib.contig_kv_attn_bf16
    good = [2 * 4 * 256, 256, 64, 48 * 128, 128, 64, 48 * 128, 128, 64, 4 * 256, 256, 64]

    def arr(v):
        return (ctypes.c_uint64 * 12)(*v)

    # q, k, v, out, lens, B, q_len, max_len, Hq, Hkv, D, scale, strides, causal, W, ws, S
    def call(strides=good, **kw):
        a = [A16, A16, A16, A16, A16, 2, 4, 48, 4, 2, 64, 0.125, arr(strides), 1, 0, A16, 2, None]
        for k, v in kw.items():
            a[{"q": 0, "out": 3, "B": 5, "n": 6, "maxlen": 7, "D": 10, "ws": 15, "S": 16}[k]] = v
        return f(*a)

    for i in range(12):                       # every stride a multiple of 16 bytes
        bad = list(good)
        bad[i] += 4
        assert call(bad) == -1, i
    huge = list(good)
    huge[4] = 1 << 28                         # 16 K rows past 2^31 bytes
    assert call(huge) == -2
    assert call(n=0) == -1
    assert call(maxlen=0) == -1
    assert call(D=96) == -2
    assert call(out=None) == -1
    assert call(ws=None) == -1                # num_splits > 1 needs the workspace
    assert call(q=A16 + 2) == -1
    assert call(B=0, out=None) == 0           # no sequences: a no-op
    assert f(A16, A16, A16, A16, A16, 2, 4, 48, 4, 2, 64, 0.125, None, 1, 0, A16, 2, None) == -1
    f8 = lib.contig_kv_attn_fp8
    odd = list(good)
    odd[4] = 72                               # 72 one-byte codes: not a multiple of 16 bytes
    assert f8(A16, A16, A16, A16, A16, 2, 4, 48, 4, 2, 64, 0.125, 1.0, 1.0, arr(odd), 1, 0, A16,
              2, None) == -1


def test_noalloc_validation(lib):
    """The static-scratch decode validates like the whole decode and rejects
    a split-K workspace larger than the scratch, before touching the GPU."""
    f = lib.paged_decode_attn_bf16_noalloc
    # q, k, v, out, bt, lens, maxb, B, Hq, Hkv, D, bs, scale, q_stride, W, S
    base = [A16, A16, A16, A16, A16, A16, 64, 2, 32, 8, 128, 16, 0.125, 4096, 0, 8, None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[{"out": 3, "S": 15, "Hq": 8, "D": 10, "q": 0, "B": 7}[k]] = v
        return f(*a)

    assert call(out=None) == -1
    assert call(Hq=5) == -1
    assert call(D=96) == -2
    assert call(S=0) == -2
    assert call(q=None) == -1
    # 2 x 32 rows x 1024 slots x 130 floats: 34 MB > 16 MiB
    assert call(S=1024) == -4
    # 4096 sequences x 32 rows at 8 slots: 545 MB
    assert call(B=4096) == -4
    assert f(None, None, None, None, None, None, 4, 0, 4, 2, 64, 16, 0.125, 256, 0, 2,
             None) == 0                         # no sequences: a no-op
