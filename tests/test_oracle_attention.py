"""Pins of the oracle's paged decode attention and its split-KV form (CPU).

* Library special case: torch.nn.functional.scaled_dot_product_attention in
  float64 on the K/V rows gathered by plain per-token indexing, with the GQA
  mapping done by torch (enable_gqa: q head h reads kv head h // G).
* The pool layout does not matter: a shuffled page pool gives bit-identical
  outputs to the same data laid out in order.
* The split-KV form gives the same result for any number of splits.
* One key returns its V row exactly; q = 0 returns the mean of V.
* A window at least as long as the sequence changes nothing; a window of W
  keys equals attention over the last W keys.
* Planted mistakes (wrong GQA mapping, a window one key too long, a page
  index off by one, a dropped split) are caught by the pins above.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import CacheGeometry, new_cache, reshape_and_cache
from oracle import attention as A
from oracle import formats as F


def _case(fmt="bf16", lens=(17, 40, 1), Hq=4, Hkv=2, D=64, bs=16, seed=0, identity=False,
          sigma=1.0, k_scale=1.0, v_scale=1.0, **geom_kw):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens)
    pages_per = (lens + bs - 1) // bs
    n_pages = int(pages_per.sum()) + 3
    maxb = int(max(1, pages_per.max()))
    perm = rng.permutation(n_pages)            # drawn either way: same q/k/v draws
    if identity:
        perm = np.arange(n_pages)
    bt = np.zeros((len(lens), maxb), np.int32)
    cur = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = perm[cur:cur + n]
        cur += n
    T = int(lens.sum())
    tok_b = np.repeat(np.arange(len(lens)), lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    tok_j = np.arange(T) - np.repeat(starts, lens)
    slots = (bt[tok_b, tok_j // bs].astype(np.int64) * bs + tok_j % bs).astype(np.int32)
    q = workloads.bf16_bits_from_f32(rng.standard_normal((len(lens), Hq, D)).astype(np.float32))
    kb = workloads.bf16_bits_from_f32((rng.standard_normal((T, Hkv, D)) * sigma).astype(np.float32))
    vb = workloads.bf16_bits_from_f32((rng.standard_normal((T, Hkv, D)) * sigma).astype(np.float32))
    geom = CacheGeometry(fmt, n_pages, bs, Hkv, D, **geom_kw)
    fill = {"bf16": 0x7FC0, "fp8": 0x7F, "nvfp4": 0x7F}[fmt]
    kc, vc = new_cache(geom, fill), new_cache(geom, fill)
    reshape_and_cache(geom, kb, vb, kc, vc, slots, k_scale=k_scale, v_scale=v_scale)
    return dict(geom=geom, q=q, kc=kc, vc=vc, bt=bt, lens=lens.astype(np.int32), kb=kb, vb=vb,
                slots=slots, tok_b=tok_b, tok_j=tok_j, Hq=Hq, maxb=maxb,
                k_scale=k_scale, v_scale=v_scale)


def _run(c, scale=0.125, window=0, seqs=None):
    return oracle.paged_decode_attention(c["geom"], c["q"], c["kc"], c["vc"], c["bt"], c["lens"],
                                         c["Hq"], scale, sliding_window=window,
                                         k_scale=c["k_scale"], v_scale=c["v_scale"], seqs=seqs)


def _sdpa_reference(c, scale, window=0):
    """torch SDPA in float64 over rows gathered token by token from the
    source (BF16) or from an independent dequantization of the written rows."""
    geom = c["geom"]
    Hq, D, bs = c["Hq"], geom.head_dim, geom.block_size
    out = []
    for b, L in enumerate(c["lens"]):
        lo = max(0, L - window) if window > 0 else 0
        q = torch.from_numpy(F.bf16_to_f64(c["q"][b]))[None, :, None, :]        # [1, Hq, 1, D]
        if geom.fmt == "bf16":
            sel = [t for t in range(len(c["tok_b"])) if c["tok_b"][t] == b and c["tok_j"][t] >= lo]
            K = F.bf16_to_f64(c["kb"][sel])
            V = F.bf16_to_f64(c["vb"][sel])
        else:
            rows = [(c["bt"][b, j // bs], j % bs) for j in range(lo, L)]
            pg = np.array([r[0] for r in rows], int)
            of = np.array([r[1] for r in rows], int)
            K = oracle.read_kv_rows(geom, c["kc"], pg, of, c["k_scale"])
            V = oracle.read_kv_rows(geom, c["vc"], pg, of, c["v_scale"])
        if K.shape[0] == 0:
            out.append(np.zeros((Hq, D)))
            continue
        Kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]   # [1, Hkv, n, D]
        Vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
        o = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, scale=scale, enable_gqa=True)
        out.append(o[0, :, 0, :].numpy())
    return np.stack(out)


CASES = [
    dict(),
    dict(lens=(1, 16, 33, 100), Hq=8, Hkv=2, D=128),
    dict(lens=(5, 64), Hq=3, Hkv=3, D=64, bs=32),
    dict(lens=(70,), Hq=16, Hkv=1, D=256, bs=64),
    dict(lens=(31, 9), Hq=8, Hkv=4, D=512),
]


@pytest.mark.parametrize("kw", CASES)
def test_matches_torch_sdpa_float64(kw):
    c = _case(**kw)
    ours = _run(c, scale=0.0883)
    ref = _sdpa_reference(c, 0.0883)
    assert np.max(np.abs(ours - ref)) < 1e-12


@pytest.mark.parametrize("window", [1, 7, 16, 17, 39, 40, 1000])
def test_window_matches_sdpa_over_last_keys(window):
    c = _case(lens=(17, 40, 3, 0))
    ours = _run(c, window=window)
    ref = _sdpa_reference(c, 0.125, window=window)
    assert np.max(np.abs(ours - ref)) < 1e-12
    if window >= 40:
        assert np.array_equal(ours, _run(c))


@pytest.mark.parametrize("fmt,kw", [
    ("fp8", dict(k_scale=np.float32(2.5 / 448), v_scale=np.float32(3.1 / 448))),
    ("fp8", dict(k_scale=np.float32(0.01), v_scale=np.float32(0.02), cache_stride=16 * 2 * 64 + 48)),
    ("nvfp4", dict()),
    ("nvfp4", dict(block_stride_bytes=1200, data_section_bytes=1040)),
])
def test_quantized_caches_match_sdpa_on_dequantized_rows(fmt, kw):
    c = _case(fmt=fmt, sigma=1.0, **kw)
    ours = _run(c)
    ref = _sdpa_reference(c, 0.125)
    assert np.max(np.abs(ours - ref)) < 1e-12
    # and the quantized result stays close to the BF16 one
    cb = _case(fmt="bf16")
    assert np.max(np.abs(ours - _run(cb))) < 0.5


def test_page_layout_does_not_matter():
    a = _case(lens=(17, 40, 100, 5), identity=False, seed=4)
    b = _case(lens=(17, 40, 100, 5), identity=True, seed=4)
    assert not np.array_equal(a["bt"], b["bt"])
    assert np.array_equal(_run(a), _run(b))


@pytest.mark.parametrize("window", [0, 20])
def test_split_count_invariance(window):
    c = _case(lens=(17, 40, 100, 5, 0), Hq=8, Hkv=2, seed=5)
    direct = _run(c, window=window)
    n = int(max((L + 15) // 16 for L in c["lens"]))
    for S in (1, 2, 3, 7, n, n + 5):
        o, m, l = oracle.split_partials(c["geom"], c["q"], c["kc"], c["vc"], c["bt"], c["lens"],
                                        c["Hq"], 0.125, S, c["maxb"], sliding_window=window)
        got = oracle.combine_partials(o, m, l)
        assert np.max(np.abs(got - direct)) < 1e-13, S


def test_split_partial_state_by_definition():
    c = _case(lens=(40,), seed=6)
    o, m, l = oracle.split_partials(c["geom"], c["q"], c["kc"], c["vc"], c["bt"], c["lens"],
                                    c["Hq"], 0.125, 1, c["maxb"])
    K = F.bf16_to_f64(c["kb"])            # tokens of the single sequence, in order
    q = F.bf16_to_f64(c["q"][0])
    for h in range(4):
        s = (K[:, h // 2] @ q[h]) * 0.125
        assert m[0, h, 0] == s.max()
        assert abs(l[0, h, 0] - np.exp(s - s.max()).sum()) < 1e-12
    assert np.max(np.abs(o[0, :, 0] - _run(c)[0])) < 1e-13
    # 3 pages over 2 splits: chunk = ceil(3/2) = 2 pages -> tokens [0,32), [32,40)
    o2, m2, l2 = oracle.split_partials(c["geom"], c["q"], c["kc"], c["vc"], c["bt"], c["lens"],
                                       c["Hq"], 0.125, 2, c["maxb"])
    s = (K[:, 0] @ q[0]) * 0.125
    assert m2[0, 0, 0] == s[:32].max() and m2[0, 0, 1] == s[32:].max()
    # 3 pages over 5 splits: splits 3 and 4 are empty
    o5, m5, l5 = oracle.split_partials(c["geom"], c["q"], c["kc"], c["vc"], c["bt"], c["lens"],
                                       c["Hq"], 0.125, 5, c["maxb"])
    assert np.all(l5[..., 3:] == 0) and np.all(np.isneginf(m5[..., 3:])) and np.all(o5[..., 3:, :] == 0)


def test_split_page_bound():
    assert A.split_page_bound(512, 16, 0) == 512
    assert A.split_page_bound(512, 16, 4096) == 257       # 4096 keys starting mid-page
    assert A.split_page_bound(512, 16, 16) == 2
    assert A.split_page_bound(512, 16, 1) == 1
    assert A.split_page_bound(8, 16, 4096) == 8
    # brute force: the most pages W consecutive keys can touch
    for bs in (16, 32):
        for W in range(1, 100):
            most = max((a + W - 1) // bs - a // bs + 1 for a in range(0, 3 * bs))
            assert A.split_page_bound(10 ** 6, bs, W) == most


def test_single_key_returns_its_value_row():
    c = _case(lens=(1, 1), Hq=4, Hkv=2, seed=7)
    out = _run(c)
    V = F.bf16_to_f64(c["vb"])           # token t = seq t here
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], V[b, h // 2])


def test_zero_query_returns_mean_of_values():
    c = _case(lens=(37,), seed=8)
    c["q"] = np.zeros_like(c["q"])
    out = _run(c)
    V = F.bf16_to_f64(c["vb"])
    for h in range(4):
        assert np.max(np.abs(out[0, h] - V[:, h // 2].mean(axis=0))) < 1e-15


def test_empty_sequence_gives_zeros():
    c = _case(lens=(0, 5))
    out = _run(c)
    assert np.all(out[0] == 0) and np.any(out[1] != 0)


def test_q_stride():
    c = _case(lens=(17, 40))
    Hq, D = 4, 64
    padded = np.full((2, Hq * D + 24), 0x7FC0, np.uint16)
    padded[:, :Hq * D] = c["q"].reshape(2, -1)
    got = oracle.paged_decode_attention(c["geom"], padded, c["kc"], c["vc"], c["bt"], c["lens"], Hq,
                                        0.125, q_stride=Hq * D + 24)
    assert np.array_equal(got, _run(c))


# ---- planted mistakes: each must be caught by one of the pins above ---------------------------

def test_planted_wrong_gqa_mapping_is_caught(monkeypatch):
    def wrong(q, K, V, scale):
        Hq, D = q.shape
        out = np.zeros((Hq, D))
        for h in range(Hq):
            g = h % K.shape[1]                    # interleaved instead of grouped
            s = (K[:, g] @ q[h]) * scale
            p = np.exp(s - s.max())
            out[h] = p @ V[:, g] / p.sum()
        return out
    monkeypatch.setattr(A, "attention_rows", wrong)
    c = _case(lens=(17, 40), Hq=4, Hkv=2)
    assert np.max(np.abs(_run(c) - _sdpa_reference(c, 0.125))) > 1e-3


def test_planted_window_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(A, "window_start", lambda L, W: max(0, L - W - 1) if W > 0 else 0)
    c = _case(lens=(17, 40))
    assert np.max(np.abs(_run(c, window=7) - _sdpa_reference(c, 0.125, window=7))) > 1e-3


def test_planted_page_offset_mistake_is_caught(monkeypatch):
    real = oracle.cache.read_kv_rows
    monkeypatch.setattr(A, "read_kv_rows",
                        lambda g, cache, pages, offs, s=1.0: real(g, cache, pages, (offs + 1) % g.block_size, s))
    a = _case(lens=(17, 40), seed=4)
    assert np.max(np.abs(_run(a) - _sdpa_reference(a, 0.125))) > 1e-3 or np.isnan(_run(a)).any()


def test_planted_dropped_split_is_caught():
    c = _case(lens=(17, 40, 100), Hq=8, Hkv=2, seed=5)
    o, m, l = oracle.split_partials(c["geom"], c["q"], c["kc"], c["vc"], c["bt"], c["lens"],
                                    c["Hq"], 0.125, 3, c["maxb"])
    l = l.copy()
    l[..., 1] = 0
    assert np.max(np.abs(oracle.combine_partials(o, m, l) - _run(c))) > 1e-3
