"""Pins of the oracle's contiguous-K/V attention (CPU).

* Library special case: torch's float64 SDPA with its bottom-right causal
  mask, on the source rows of every sequence.
* The layout does not matter: sequence-major (b, l, h, d) and head-major
  (b, h, l, d) K/V, and the same for q, give bit-identical outputs.
* A paged cache holding the same rows gives bit-identical outputs (the
  paged-versus-contiguous invariant).
* FP8 codes: the same as the paged FP8 cache written with the same scale.
* A planted stride mistake (token and head strides swapped) is caught.
"""
import numpy as np
import pytest
import torch
from torch.nn.attention.bias import causal_lower_right

import oracle
import workloads
from oracle import attention as A
from oracle import formats as F

pytestmark = pytest.mark.filterwarnings("ignore:Lower right causal bias")


def _source(lens, q_len, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    rows = [(workloads.bf16_bits_from_f32(rng.standard_normal((L, Hkv, D)).astype(np.float32)),
             workloads.bf16_bits_from_f32(rng.standard_normal((L, Hkv, D)).astype(np.float32)))
            for L in lens]
    q = workloads.bf16_bits_from_f32(rng.standard_normal((len(lens), q_len, Hq, D)).astype(np.float32))
    return rows, q


def _lay_out(rows, layout, Lmax, fill, dtype=np.uint16):
    """[B, Lmax, Hkv, D] ("blhd") or [B, Hkv, Lmax, D] ("bhld") with its strides."""
    B = len(rows)
    Hkv, D = rows[0].shape[1], rows[0].shape[2]
    t = np.full((B, Lmax, Hkv, D), fill, dtype)
    for b, r in enumerate(rows):
        t[b, :len(r)] = r
    if layout == "bhld":
        t = np.ascontiguousarray(t.transpose(0, 2, 1, 3))
        return t, (Hkv * Lmax * D, D, Lmax * D)
    return t, (Lmax * Hkv * D, Hkv * D, D)


def _q_layout(q, layout):
    B, n, Hq, D = q.shape
    if layout == "bhld":
        return np.ascontiguousarray(q.transpose(0, 2, 1, 3)), (Hq * n * D, D, n * D)
    return q, (n * Hq * D, Hq * D, D)


def _run(fmt, q, qs, k, ks, v, vs, lens, Hq, Hkv, D, n, causal=True, window=0, k_scale=1.0,
         v_scale=1.0):
    return oracle.contiguous_attention(fmt, q, k, v, lens, Hq, Hkv, D, n, 0.0883, qs, ks, vs,
                                       causal=causal, sliding_window=window, k_scale=k_scale,
                                       v_scale=v_scale)


@pytest.mark.parametrize("lens,n,Hq,Hkv,D", [((17, 40), 4, 4, 2, 64), ((1, 33, 100), 3, 8, 2, 128),
                                            ((5, 64), 6, 3, 3, 64), ((3, 20), 6, 4, 2, 64)])
def test_matches_sdpa_lower_right(lens, n, Hq, Hkv, D):
    rows, q = _source(lens, n, Hq, Hkv, D, seed=len(lens) + n)
    Lmax = max(lens) + 5
    k, ks = _lay_out([r[0] for r in rows], "blhd", Lmax, 0x7FC0)
    v, vs = _lay_out([r[1] for r in rows], "blhd", Lmax, 0x7FC0)
    qq, qs = _q_layout(q, "blhd")
    ours = _run("bf16", qq, qs, k, ks, v, vs, np.array(lens), Hq, Hkv, D, n)
    for b, L in enumerate(lens):
        K = F.bf16_to_f64(rows[b][0]).transpose(1, 0, 2)[None]
        V = F.bf16_to_f64(rows[b][1]).transpose(1, 0, 2)[None]
        qt = F.bf16_to_f64(q[b]).transpose(1, 0, 2)[None]
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qt.copy()), torch.from_numpy(K.copy()), torch.from_numpy(V.copy()),
            attn_mask=causal_lower_right(n, L), scale=0.0883, enable_gqa=True)
        o = o[0].numpy().transpose(1, 0, 2)
        for i in range(n):
            if L - n + i < 0:
                assert np.all(ours[b, i] == 0)
            else:
                assert np.max(np.abs(ours[b, i] - o[i])) < 1e-12


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 7), (False, 0), (False, 9)])
def test_layouts_and_paged_twin(causal, window):
    lens, n, Hq, Hkv, D, bs = (17, 40, 0, 3), 4, 8, 2, 64, 16
    rows, q = _source(lens, n, Hq, Hkv, D, seed=2)
    Lmax = 48
    outs = []
    for kl in ("blhd", "bhld"):
        for ql in ("blhd", "bhld"):
            k, ks = _lay_out([r[0] for r in rows], kl, Lmax, 0x7FC0)
            v, vs = _lay_out([r[1] for r in rows], kl, Lmax, 0x7FC0)
            qq, qs = _q_layout(q, ql)
            outs.append(_run("bf16", qq, qs, k, ks, v, vs, np.array(lens), Hq, Hkv, D, n,
                             causal=causal, window=window))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    # the same rows in a paged cache behind a shuffled block table
    rng = np.random.default_rng(3)
    maxb = Lmax // bs
    perm = rng.permutation(len(lens) * maxb + 2)
    bt = perm[:len(lens) * maxb].reshape(len(lens), maxb).astype(np.int32)
    geom = oracle.CacheGeometry("bf16", len(perm), bs, Hkv, D)
    kc, vc = oracle.new_cache(geom, 0x7FC0), oracle.new_cache(geom, 0x7FC0)
    for b, L in enumerate(lens):
        j = np.arange(L)
        slots = (bt[b, j // bs].astype(np.int64) * bs + j % bs).astype(np.int32)
        oracle.reshape_and_cache(geom, rows[b][0], rows[b][1], kc, vc, slots)
    paged = oracle.paged_prefill_attention(geom, q, kc, vc, bt, np.array(lens, np.int32), Hq, n,
                                           0.0883, causal=causal, sliding_window=window)
    assert np.array_equal(paged, outs[0])


def test_fp8_codes_match_the_paged_fp8_cache():
    lens, n, Hq, Hkv, D, bs = (17, 40), 3, 4, 2, 128, 16
    rows, q = _source(lens, n, Hq, Hkv, D, seed=4)
    ksc, vsc = np.float32(0.011), np.float32(0.007)
    Lmax = 48
    kb, _ = _lay_out([r[0] for r in rows], "blhd", Lmax, 0)
    vb, _ = _lay_out([r[1] for r in rows], "blhd", Lmax, 0)
    kcodes = oracle.e4m3_encode(F.bf16_to_f64(kb).astype(np.float32), ksc)
    vcodes = oracle.e4m3_encode(F.bf16_to_f64(vb).astype(np.float32), vsc)
    strides = (Lmax * Hkv * D, Hkv * D, D)
    qq, qs = _q_layout(q, "blhd")
    ours = _run("fp8", qq, qs, kcodes, strides, vcodes, strides, np.array(lens), Hq, Hkv, D, n,
                k_scale=ksc, v_scale=vsc)
    maxb = Lmax // bs
    bt = np.arange(len(lens) * maxb, dtype=np.int32).reshape(len(lens), maxb)
    geom = oracle.CacheGeometry("fp8", len(lens) * maxb, bs, Hkv, D)
    kc, vc = oracle.new_cache(geom, 0), oracle.new_cache(geom, 0)
    for b, L in enumerate(lens):
        j = np.arange(L)
        slots = (bt[b, j // bs].astype(np.int64) * bs + j % bs).astype(np.int32)
        oracle.reshape_and_cache(geom, rows[b][0], rows[b][1], kc, vc, slots, k_scale=ksc,
                                 v_scale=vsc)
    paged = oracle.paged_prefill_attention(geom, q, kc, vc, bt, np.array(lens, np.int32), Hq, n,
                                           0.0883, k_scale=ksc, v_scale=vsc)
    assert np.array_equal(paged, ours)


def test_planted_stride_swap_is_caught():
    lens, n, Hq, Hkv, D = (17, 40), 2, 4, 2, 64
    rows, q = _source(lens, n, Hq, Hkv, D, seed=5)
    k, ks = _lay_out([r[0] for r in rows], "blhd", 40, 0)
    v, vs = _lay_out([r[1] for r in rows], "blhd", 40, 0)
    qq, qs = _q_layout(q, "blhd")
    good = _run("bf16", qq, qs, k, ks, v, vs, np.array(lens), Hq, Hkv, D, n)
    bad_ks = (ks[0], ks[2], ks[1])
    bad = _run("bf16", qq, qs, k, bad_ks, v, vs, np.array(lens), Hq, Hkv, D, n)
    assert np.max(np.abs(bad - good)) > 1e-3
