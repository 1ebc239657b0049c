"""Pins of the oracle's multi-token paged attention (CPU).

* Library special case: torch's scaled_dot_product_attention in float64 with
  torch's own bottom-right-aligned causal mask (causal_lower_right), whose
  query i of q_len sits at key position kv_len - q_len + i, on K/V rows
  gathered token by token from the source rows (BF16 caches) or from the
  written cache rows (FP8 / NVFP4), GQA mapped by torch (enable_gqa).
* Not causal: every query token gets what a one-token decode of the sequence
  gives (torch SDPA without a mask, and the pinned decode oracle).
* One query token: identical to the pinned decode oracle, causal or not.
* q = 0 gives the mean of V over exactly the keys the token attends,
  window included, from the source rows (a closed form).
* Tokens at negative positions (q_len > seq_len) attend nothing: zeros.
* Planted mistakes (causal limit off by one, query rows of the wrong token,
  window measured from the sequence end instead of the token) are caught.
"""
import numpy as np
import pytest
import torch
from torch.nn.attention.bias import causal_lower_right

import oracle
import workloads
from oracle import CacheGeometry, new_cache, reshape_and_cache
from oracle import attention as A
from oracle import formats as F

# rows of tokens at negative positions are compared against zeros, not SDPA
pytestmark = pytest.mark.filterwarnings("ignore:Lower right causal bias")


def _case(fmt="bf16", lens=(17, 40), q_len=4, Hq=4, Hkv=2, D=64, bs=16, seed=0, sigma=1.0,
          k_scale=1.0, v_scale=1.0):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens)
    pages_per = (lens + bs - 1) // bs
    n_pages = int(pages_per.sum()) + 3
    maxb = int(max(1, pages_per.max()))
    perm = rng.permutation(n_pages)
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
    q = workloads.bf16_bits_from_f32(rng.standard_normal((len(lens), q_len, Hq, D)).astype(np.float32))
    kb = workloads.bf16_bits_from_f32((rng.standard_normal((T, Hkv, D)) * sigma).astype(np.float32))
    vb = workloads.bf16_bits_from_f32((rng.standard_normal((T, Hkv, D)) * sigma).astype(np.float32))
    geom = CacheGeometry(fmt, n_pages, bs, Hkv, D)
    fill = {"bf16": 0x7FC0, "fp8": 0x7F, "nvfp4": 0x7F}[fmt]
    kc, vc = new_cache(geom, fill), new_cache(geom, fill)
    reshape_and_cache(geom, kb, vb, kc, vc, slots, k_scale=k_scale, v_scale=v_scale)
    return dict(geom=geom, q=q, kc=kc, vc=vc, bt=bt, lens=lens.astype(np.int32), kb=kb, vb=vb,
                tok_b=tok_b, tok_j=tok_j, Hq=Hq, q_len=q_len, k_scale=k_scale, v_scale=v_scale)


def _run(c, causal=True, window=0, scale=0.125, **kw):
    return oracle.paged_prefill_attention(c["geom"], c["q"], c["kc"], c["vc"], c["bt"], c["lens"],
                                          c["Hq"], c["q_len"], scale, causal=causal,
                                          sliding_window=window, k_scale=c["k_scale"],
                                          v_scale=c["v_scale"], **kw)


def _rows(c, b):
    """All keys and values of sequence b in position order, float64."""
    geom = c["geom"]
    L = int(c["lens"][b])
    if geom.fmt == "bf16":
        sel = [t for t in range(len(c["tok_b"])) if c["tok_b"][t] == b]
        sel.sort(key=lambda t: c["tok_j"][t])
        return F.bf16_to_f64(c["kb"][sel]), F.bf16_to_f64(c["vb"][sel])
    bs = geom.block_size
    pg = np.array([c["bt"][b, j // bs] for j in range(L)], int)
    of = np.array([j % bs for j in range(L)], int)
    return (oracle.read_kv_rows(geom, c["kc"], pg, of, c["k_scale"]),
            oracle.read_kv_rows(geom, c["vc"], pg, of, c["v_scale"]))


def _sdpa_causal(c, scale):
    """torch SDPA float64 with torch's bottom-right causal mask; rows of
    tokens at negative positions (no key) come back as None."""
    out = []
    n = c["q_len"]
    for b, L in enumerate(c["lens"]):
        K, V = _rows(c, b)
        q = torch.from_numpy(F.bf16_to_f64(c["q"][b]).transpose(1, 0, 2).copy())[None]  # [1,Hq,n,D]
        Kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
        Vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
        o = torch.nn.functional.scaled_dot_product_attention(
            q, Kt, Vt, attn_mask=causal_lower_right(n, int(L)), scale=scale, enable_gqa=True)
        o = o[0].numpy().transpose(1, 0, 2)                      # [n, Hq, D]
        out.append([o[i] if int(L) - n + i >= 0 else None for i in range(n)])
    return out


CASES = [
    dict(),
    dict(lens=(1, 16, 33, 100), q_len=3, Hq=8, Hkv=2, D=128),
    dict(lens=(5, 64), q_len=16, Hq=3, Hkv=3, bs=32),
    dict(lens=(70,), q_len=9, Hq=16, Hkv=1, D=256, bs=64),
    dict(lens=(31, 9), q_len=2, Hq=8, Hkv=4, D=512),
    dict(lens=(3, 20), q_len=6),                  # q_len > L: early tokens attend nothing
]


@pytest.mark.parametrize("kw", CASES)
def test_causal_matches_sdpa_lower_right_float64(kw):
    c = _case(**kw)
    ours = _run(c, scale=0.0883)
    ref = _sdpa_causal(c, 0.0883)
    for b in range(len(c["lens"])):
        for i in range(c["q_len"]):
            if ref[b][i] is None:
                assert np.all(ours[b, i] == 0)
            else:
                assert np.max(np.abs(ours[b, i] - ref[b][i])) < 1e-12, (b, i)


@pytest.mark.parametrize("fmt,kw", [
    ("fp8", dict(k_scale=np.float32(2.5 / 448), v_scale=np.float32(3.1 / 448))),
    ("nvfp4", dict()),
])
def test_quantized_causal_matches_sdpa(fmt, kw):
    c = _case(fmt=fmt, lens=(17, 40, 2), q_len=5, **kw)
    ours = _run(c)
    ref = _sdpa_causal(c, 0.125)
    for b in range(3):
        for i in range(5):
            if ref[b][i] is None:
                assert np.all(ours[b, i] == 0)
            else:
                assert np.max(np.abs(ours[b, i] - ref[b][i])) < 1e-12


@pytest.mark.parametrize("window", [0, 5, 17])
def test_not_causal_is_decode_of_every_token(window):
    c = _case(lens=(17, 40, 0), q_len=3)
    ours = _run(c, causal=False, window=window)
    for i in range(3):
        dec = oracle.paged_decode_attention(c["geom"], np.ascontiguousarray(c["q"][:, i]), c["kc"],
                                            c["vc"], c["bt"], c["lens"], c["Hq"], 0.125,
                                            sliding_window=window)
        assert np.array_equal(ours[:, i], dec)
    # and against SDPA without a mask
    for b, L in enumerate(c["lens"][:2]):
        K, V = _rows(c, b)
        lo = A.window_start(int(L), window)
        q = torch.from_numpy(F.bf16_to_f64(c["q"][b]).transpose(1, 0, 2).copy())[None]
        Kt = torch.from_numpy(np.ascontiguousarray(K[lo:].transpose(1, 0, 2)))[None]
        Vt = torch.from_numpy(np.ascontiguousarray(V[lo:].transpose(1, 0, 2)))[None]
        o = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, scale=0.125,
                                                             enable_gqa=True)
        assert np.max(np.abs(ours[b] - o[0].numpy().transpose(1, 0, 2))) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [0, 1, 7, 40])
def test_one_token_is_decode(causal, window):
    c = _case(lens=(17, 40, 1, 0), q_len=1)
    ours = _run(c, causal=causal, window=window)
    dec = oracle.paged_decode_attention(c["geom"], np.ascontiguousarray(c["q"][:, 0]), c["kc"],
                                        c["vc"], c["bt"], c["lens"], c["Hq"], 0.125,
                                        sliding_window=window)
    assert np.array_equal(ours[:, 0], dec)


@pytest.mark.parametrize("window", [0, 1, 3, 8, 20])
def test_zero_query_is_mean_over_the_attended_keys(window):
    """q = 0: every logit is 0, so token i returns the plain mean of V over
    keys max(0, p - W + 1) .. p (p = L - q_len + i), read from the source rows."""
    c = _case(lens=(17, 40, 4), q_len=6, seed=3)
    c["q"] = np.zeros_like(c["q"])
    ours = _run(c, window=window)
    for b, L in enumerate(c["lens"]):
        _, V = _rows(c, b)
        for i in range(6):
            p = int(L) - 6 + i
            if p < 0:
                assert np.all(ours[b, i] == 0)
                continue
            first = max(0, p - window + 1) if window > 0 else 0
            for h in range(4):
                want = V[first:p + 1, h // 2].mean(axis=0)
                assert np.max(np.abs(ours[b, i, h] - want)) < 1e-15, (b, i, window)


@pytest.mark.parametrize("window", [0, 6])
def test_causal_token_is_decode_of_the_prefix(window):
    """Token i of a causal block equals a decode whose sequence ends at the
    token's position."""
    c = _case(lens=(17, 40), q_len=4, seed=9)
    ours = _run(c, window=window)
    for i in range(4):
        lens_i = (c["lens"] - 4 + i + 1).astype(np.int32)
        dec = oracle.paged_decode_attention(c["geom"], np.ascontiguousarray(c["q"][:, i]), c["kc"],
                                            c["vc"], c["bt"], lens_i, c["Hq"], 0.125,
                                            sliding_window=window)
        assert np.array_equal(ours[:, i], dec)


def test_strided_query_rows():
    c = _case(lens=(17, 40), q_len=3)
    Hq, D = 4, 64
    tok_stride, seq_stride = Hq * D + 40, 3 * (Hq * D + 40) + 8
    padded = np.full(2 * seq_stride, 0x7FC0, np.uint16)
    for b in range(2):
        for i in range(3):
            s = b * seq_stride + i * tok_stride
            padded[s:s + Hq * D] = c["q"][b, i].reshape(-1)
    got = _run(dict(c, q=padded), q_stride=seq_stride, q_token_stride=tok_stride)
    assert np.array_equal(got, _run(c))


def test_state_by_definition():
    c = _case(lens=(40,), q_len=3, seed=6)
    out, m, l = _run(c, return_state=True)
    K, _ = _rows(c, 0)
    q = F.bf16_to_f64(c["q"][0])
    for i in range(3):
        for h in range(4):
            s = (K[:38 + i, h // 2] @ q[i, h]) * 0.125
            assert m[0, i, h] == s.max()
            assert abs(l[0, i, h] - np.exp(s - s.max()).sum()) < 1e-12
    c2 = _case(lens=(2,), q_len=4)
    _, m2, l2 = _run(c2, return_state=True)
    assert np.all(np.isneginf(m2[0, :2])) and np.all(l2[0, :2] == 0) and np.all(l2[0, 2:] > 0)


def test_query_range_brute_force():
    """The attended set of every token, against a key-by-key membership test
    written from the causal and window rules."""
    for L in range(0, 40):
        for n in (1, 2, 5, 17):
            for W in (0, 1, 3, 16):
                for i in range(n):
                    p = L - n + i
                    want = [j for j in range(L) if j <= p and (W == 0 or j > p - W)]
                    lo, hi = A.query_range(L, n, i, True, W)
                    assert list(range(lo, hi)) == want, (L, n, i, W)
                    lo, hi = A.query_range(L, n, i, False, W)
                    assert list(range(lo, hi)) == [j for j in range(L) if W == 0 or j >= L - W]


# ---- planted mistakes: each must be caught by one of the pins above ---------------------------

def test_planted_causal_off_by_one_is_caught(monkeypatch):
    real = A.query_range
    monkeypatch.setattr(A, "query_range",
                        lambda L, n, i, causal, W: real(L, n, i - 1, causal, W) if i > 0
                        else real(L, n, i, causal, W))
    c = _case(lens=(17, 40), q_len=4)
    ours = _run(c)
    ref = _sdpa_causal(c, 0.125)
    assert max(np.max(np.abs(ours[b, i] - ref[b][i])) for b in range(2) for i in range(4)) > 1e-3


def test_planted_wrong_token_rows_are_caught(monkeypatch):
    real = A._prefill_q_rows
    monkeypatch.setattr(A, "_prefill_q_rows",
                        lambda q, b, i, Hq, D, qs, ts: real(q, b, 0, Hq, D, qs, ts))
    c = _case(lens=(17, 40), q_len=4)
    ours = _run(c)
    ref = _sdpa_causal(c, 0.125)
    assert max(np.max(np.abs(ours[b, i] - ref[b][i])) for b in range(2) for i in range(4)) > 1e-3


def test_planted_window_from_sequence_end_is_caught(monkeypatch):
    real = A.query_range
    def wrong(L, n, i, causal, W):
        lo, hi = real(L, n, i, causal, 0)
        return (max(lo, L - W) if W > 0 else lo), hi
    monkeypatch.setattr(A, "query_range", wrong)
    c = _case(lens=(17, 40), q_len=6, seed=3)
    c["q"] = np.zeros_like(c["q"])
    ours = _run(c, window=3)
    _, V = _rows(c, 1)
    assert np.max(np.abs(ours[1, 0, 0] - V[32:35, 0].mean(axis=0))) > 1e-3
