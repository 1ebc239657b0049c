"""Pins of the oracle's cache writes and absmax (CPU only).

Each layout is checked by reading the written pool back through an
independent view built with numpy reshapes of the page bytes (not through the
oracle's own index formulas), against the row encoders applied token by
token; untouched bytes (unused slots, padding between sections and pages)
must keep their sentinel value.
"""
import numpy as np
import pytest

import oracle
from oracle import CacheGeometry, new_cache, reshape_and_cache
from oracle import formats as F


def _setup(fmt, bs=16, Hkv=2, D=64, pages=6, ntok=50, seed=0, **kw):
    rng = np.random.default_rng(seed)
    geom = CacheGeometry(fmt, pages, bs, Hkv, D, **kw)
    slots = rng.permutation(pages * bs)[:ntok].astype(np.int32)
    key = (rng.standard_normal((ntok, Hkv, D)) * 2).astype(np.float32)
    val = (rng.standard_normal((ntok, Hkv, D)) * 0.5).astype(np.float32)
    import workloads
    kb = workloads.bf16_bits_from_f32(key)
    vb = workloads.bf16_bits_from_f32(val)
    return geom, slots, kb, vb


def _unwritten_slots(geom, slots):
    all_slots = np.arange(geom.num_pages * geom.block_size)
    return np.setdiff1d(all_slots, slots)


def test_bf16_write_reads_back_through_reshape():
    geom, slots, kb, vb = _setup("bf16")
    kc, vc = new_cache(geom, 0x7FC0), new_cache(geom, 0x7FC0)
    reshape_and_cache(geom, kb, vb, kc, vc, slots)
    kview = kc.reshape(geom.num_pages, geom.block_size, geom.num_kv_heads, geom.head_dim)
    vview = vc.reshape(geom.num_pages, geom.block_size, geom.num_kv_heads, geom.head_dim)
    for t, s in enumerate(slots):
        assert np.array_equal(kview[s // 16, s % 16], kb[t])
        assert np.array_equal(vview[s // 16, s % 16], vb[t])
    for s in _unwritten_slots(geom, slots):
        assert np.all(kview[s // 16, s % 16] == 0x7FC0)


def test_bf16_write_source_stride_and_negative_slots():
    geom, slots, kb, vb = _setup("bf16", ntok=20)
    # source rows padded to a stride of Hkv*D + 40 elements
    stride = geom.num_kv_heads * geom.head_dim + 40
    src_k = np.full((20, stride), 0x1234, np.uint16)
    src_k[:, :geom.num_kv_heads * geom.head_dim] = kb.reshape(20, -1)
    src_v = np.full((20, stride), 0x1234, np.uint16)
    src_v[:, :geom.num_kv_heads * geom.head_dim] = vb.reshape(20, -1)
    slots = slots.copy()
    slots[[3, 7]] = -1
    kc, vc = new_cache(geom, 0), new_cache(geom, 0)
    reshape_and_cache(geom, src_k, src_v, kc, vc, slots, key_stride=stride, value_stride=stride)
    kview = kc.reshape(geom.num_pages, 16, geom.num_kv_heads, geom.head_dim)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kview[s // 16, s % 16], kb[t])
    assert np.count_nonzero(kc) == np.count_nonzero(kb[np.array(slots) >= 0])


@pytest.mark.parametrize("stride_pad", [0, 100])
def test_fp8_write_layout(stride_pad):
    bs, Hkv, D = 16, 2, 64
    packed = bs * Hkv * D
    geom, slots, kb, vb = _setup("fp8", bs=bs, Hkv=Hkv, D=D, cache_stride=packed + stride_pad)
    k_scale, v_scale = np.float32(0.05), np.float32(0.0071)
    kc, vc = new_cache(geom, 0x7F), new_cache(geom, 0x7F)
    reshape_and_cache(geom, kb, vb, kc, vc, slots, k_scale=k_scale, v_scale=v_scale)
    kpages = kc.reshape(geom.num_pages, packed + stride_pad)
    kview = kpages[:, :packed].reshape(geom.num_pages, bs, Hkv, D)
    for t, s in enumerate(slots):
        row = F.bf16_to_f64(kb[t]).astype(np.float32)
        assert np.array_equal(kview[s // bs, s % bs], F.e4m3_encode(row, k_scale))
    assert np.all(kpages[:, packed:] == 0x7F)
    # decoding the written codes gives the quantized values back
    rows = oracle.read_kv_rows(geom, kc, slots // bs, slots % bs, k_scale)
    exact = F.bf16_to_f64(kb)
    assert np.max(np.abs(rows - exact)) <= 448 * float(k_scale) * 2 ** -4 + 1e-12


@pytest.mark.parametrize("pad", [(0, 0), (64, 32)])
def test_nvfp4_write_layout(pad):
    bs, Hkv, D = 16, 2, 64
    data = bs * Hkv * D // 2 + pad[0]
    stride = data + bs * Hkv * D // 16 + pad[1]
    geom, slots, kb, vb = _setup("nvfp4", bs=bs, Hkv=Hkv, D=D,
                                 block_stride_bytes=stride, data_section_bytes=data)
    kc, vc = new_cache(geom, 0xEE), new_cache(geom, 0xEE)
    reshape_and_cache(geom, kb, vb, kc, vc, slots)
    pages = kc.reshape(geom.num_pages, stride)
    dview = pages[:, :bs * Hkv * D // 2].reshape(geom.num_pages, bs, Hkv, D // 2)
    sview = pages[:, data:data + bs * Hkv * D // 16].reshape(geom.num_pages, bs, Hkv, D // 16)
    for t, s in enumerate(slots):
        row = F.bf16_to_f64(kb[t]).astype(np.float32).reshape(Hkv, D // 16, 16)
        codes, sc = F.nvfp4_encode_groups(row)
        codes = codes.reshape(Hkv, D)
        byte = dview[s // bs, s % bs]
        assert np.array_equal(byte & 0xF, codes[:, 0::2])
        assert np.array_equal(byte >> 4, codes[:, 1::2])
        assert np.array_equal(sview[s // bs, s % bs], sc)
    # padding between the sections and after the scales is untouched
    assert np.all(pages[:, bs * Hkv * D // 2:data] == 0xEE)
    assert np.all(pages[:, data + bs * Hkv * D // 16:] == 0xEE)
    # unwritten slots keep the sentinel in both sections
    for s in _unwritten_slots(geom, slots):
        assert np.all(dview[s // bs, s % bs] == 0xEE) and np.all(sview[s // bs, s % bs] == 0xEE)


@pytest.mark.parametrize("pad", [(0, 0), (64, 32)])
def test_read_rows_nvfp4_exact_through_reshape_view(pad):
    """The NVFP4 branch of read_kv_rows equals, bit for bit, the rows
    gathered through a reshape view of the page bytes (codes unpacked low
    nibble first, scales from their own section view) and decoded by
    nvfp4_decode_groups: no index formula of read_kv_rows is reused."""
    bs, Hkv, D = 16, 2, 128
    data = bs * Hkv * D // 2 + pad[0]
    stride = data + bs * Hkv * D // 16 + pad[1]
    geom, slots, kb, vb = _setup("nvfp4", bs=bs, Hkv=Hkv, D=D, pages=7, ntok=80, seed=9,
                                 block_stride_bytes=stride, data_section_bytes=data)
    kc, vc = new_cache(geom, 0xEE), new_cache(geom, 0xEE)
    reshape_and_cache(geom, kb, vb, kc, vc, slots)
    got = oracle.read_kv_rows(geom, kc, slots // bs, slots % bs)
    pages = kc.reshape(geom.num_pages, stride)
    dview = pages[:, :bs * Hkv * D // 2].reshape(geom.num_pages, bs, Hkv, D // 2)
    sview = pages[:, data:data + bs * Hkv * D // 16].reshape(geom.num_pages, bs, Hkv, D // 16)
    byte = dview[slots // bs, slots % bs]                      # [n, Hkv, D/2]
    codes = np.stack([byte & 0xF, byte >> 4], axis=-1).reshape(len(slots), Hkv, D // 16, 16)
    want = F.nvfp4_decode_groups(codes, sview[slots // bs, slots % bs]).reshape(len(slots), Hkv, D)
    assert np.array_equal(got, want)
    # and each row is what the group encoder gives for its BF16 source
    for t in range(len(slots)):
        src = F.bf16_to_f64(kb[t]).astype(np.float32).reshape(Hkv, D // 16, 16)
        c, sc = F.nvfp4_encode_groups(src)
        assert np.array_equal(got[t], F.nvfp4_decode_groups(c, sc).reshape(Hkv, D))


def test_read_rows_bf16_exact_through_reshape_view():
    geom, slots, kb, vb = _setup("bf16", Hkv=4, D=128, pages=5, ntok=60, seed=4)
    kc, vc = new_cache(geom, 0x7FC0), new_cache(geom, 0x7FC0)
    reshape_and_cache(geom, kb, vb, kc, vc, slots)
    got = oracle.read_kv_rows(geom, vc, slots // 16, slots % 16)
    view = vc.reshape(geom.num_pages, 16, 4, 128)
    assert np.array_equal(got, F.bf16_to_f64(view[slots // 16, slots % 16]))
    assert np.array_equal(got, F.bf16_to_f64(vb))


def test_read_rows_decodes_fp8_as_code_times_scale():
    geom = CacheGeometry("fp8", 1, 16, 1, 16)
    kc = np.arange(256, dtype=np.uint8)
    rows = oracle.read_kv_rows(geom, kc, np.zeros(16, int), np.arange(16), 0.25)
    expect = F.e4m3_decode(np.arange(256, dtype=np.uint8)).reshape(16, 1, 16) * 0.25
    assert np.array_equal(np.isnan(rows), np.isnan(expect))
    ok = ~np.isnan(expect)
    assert np.array_equal(rows[ok], expect[ok])


def test_bf16_absmax():
    rng = np.random.default_rng(3)
    import workloads
    x = workloads.bf16_bits_from_f32(rng.standard_normal(10000).astype(np.float32) * 3)
    ref = np.max(np.abs(F.bf16_to_f64(x)))
    assert oracle.bf16_absmax(x) == np.float32(ref)
    assert oracle.bf16_absmax(x, out_in=100.0) == np.float32(100.0)
    y = x.copy()
    y[5] = 0x7FC0                     # NaN is ignored
    y[6] = 0xFFC0
    assert oracle.bf16_absmax(y) == oracle.bf16_absmax(np.delete(x, [5, 6]))
    assert oracle.bf16_absmax(np.array([0x8000], np.uint16)) == 0.0   # |-0| = 0
    assert oracle.bf16_absmax(np.array([0xC2C8], np.uint16)) == 100.0  # -100
