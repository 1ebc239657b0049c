"""GPU parity of multi-token paged attention (query blocks of q_len tokens
per sequence, causal or not), called through the C ABI, against the CPU
oracle on the same seeded inputs; atol = rtol = 1e-2 on the BF16 outputs."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_splitk_amd as pkd
import workloads
from gpu_cases import (DeviceKV, assert_close, fp8_scales, full_size_reference, geometry,
                       oracle_pools,
                       oracle_prefill, pool_to_np)

pytestmark = pytest.mark.gpu


def _num_cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _small_fp8_scales(w):
    k = oracle.bf16_absmax(w.k_bits) / np.float32(448.0)
    v = oracle.bf16_absmax(w.v_bits) / np.float32(448.0)
    return np.float32(k), np.float32(v)


def _setup(fmt, lens, Hq, Hkv, D, bs, window, seed):
    w = workloads.make_workload("tiny", lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                block_size=bs, sliding_window=window, kv_dtype=fmt, seed=seed)
    geom = geometry(w)
    ks, vs = _small_fp8_scales(w) if fmt == "fp8" else (1.0, 1.0)
    d = DeviceKV(w, geom, ks, vs)
    kc, vc = oracle_pools(w, geom, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(pool_to_np(d.k, fmt), kc)
    return w, geom, d, kc, vc, ks, vs


CASES = [
    # fmt, lens, q_len, Hq, Hkv, D, bs, causal, window, S
    ("bf16", (17, 40), 4, 4, 2, 64, 16, 1, 0, 1),
    ("bf16", (17, 40), 4, 4, 2, 64, 16, 1, 0, 3),
    ("bf16", (1, 15, 16, 17, 100, 300), 4, 32, 8, 128, 16, 1, 0, 1),     # 16 columns: one chunk
    ("bf16", (1, 15, 16, 17, 100, 300), 4, 32, 8, 128, 16, 1, 0, 5),
    ("bf16", (33, 257, 1000), 8, 32, 8, 128, 16, 1, 0, 7),               # 32 columns: two chunks
    ("bf16", (33, 257, 1000), 3, 32, 8, 128, 16, 0, 0, 4),               # not causal
    ("bf16", (2, 5, 77, 130), 6, 4, 4, 64, 32, 1, 0, 2),                 # L < q_len
    ("bf16", (64, 200), 17, 16, 1, 256, 64, 1, 0, 3),                    # 272 columns
    ("bf16", (50, 180), 2, 8, 1, 512, 16, 1, 0, 2),                      # split head dim
    ("bf16", (50, 180), 5, 8, 1, 512, 16, 1, 0, 1),
    ("bf16", (90, 400, 17), 5, 6, 2, 64, 16, 1, 37, 3),                  # causal window
    ("bf16", (90, 400, 17), 5, 6, 2, 64, 128, 0, 37, 2),                 # plain window
    ("bf16", (90, 400, 17), 33, 6, 2, 64, 16, 1, 20, 4),                 # window < q_len
    ("bf16", (0, 5, 40), 8, 8, 2, 64, 16, 1, 0, 1),                     # two chunks per wave
    ("bf16", (0, 5, 40, 300), 12, 8, 2, 128, 16, 1, 0, 4),              # three chunks: 2 + 1
    ("bf16", (100, 700), 16, 32, 8, 128, 16, 1, 100, 3),                # four chunks, window
    ("bf16", (0, 5, 40), 12, 8, 2, 64, 16, 1, 0, 1),                    # waves sharing tiles
    ("bf16", (1, 33, 530), 24, 16, 2, 128, 32, 1, 0, 1),                # 192 columns, one piece
    ("bf16", (1, 33, 530), 24, 16, 2, 128, 32, 1, 70, 6),
    ("bf16", (64, 200), 9, 16, 1, 256, 16, 0, 0, 1),                    # head_dim 256, shared
    ("bf16", (0, 64, 200), 2, 16, 1, 256, 16, 1, 0, 3),                 # two waves share, D 256
    ("fp8", (1, 17, 300, 1000), 2, 16, 8, 256, 16, 1, 0, 3),
    ("fp8", (1, 17, 300, 1000), 3, 16, 8, 256, 16, 1, 129, 5),
    ("fp8", (40, 333), 4, 8, 1, 128, 16, 1, 60, 2),
    ("fp8", (40, 100), 2, 16, 2, 512, 16, 1, 0, 2),
    ("fp8", (0, 1, 2, 700), 4, 16, 8, 256, 16, 1, 0, 4),
    ("nvfp4", (1, 17, 300, 1000), 2, 16, 2, 512, 16, 1, 0, 3),
    ("nvfp4", (1, 17, 300, 700), 3, 16, 2, 512, 16, 1, 200, 4),
    ("nvfp4", (40, 333), 4, 8, 2, 128, 16, 1, 0, 2),
    ("nvfp4", (40, 333), 4, 8, 2, 64, 32, 0, 0, 1),
    ("nvfp4", (0, 1, 2, 700), 8, 16, 2, 512, 16, 1, 0, 4),
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"{c[0]}-n{c[2]}-D{c[5]}-G{c[3] // c[4]}-bs{c[6]}-{'c' if c[7] else 'nc'}-W{c[8]}-S{c[9]}"
    for c in CASES])
def test_prefill_matches_oracle(case):
    fmt, lens, n, Hq, Hkv, D, bs, causal, window, S = case
    w, geom, d, kc, vc, ks, vs = _setup(fmt, lens, Hq, Hkv, D, bs, window, seed=D + n + S)
    q = workloads.query_block(w, n, seed=S)
    got = d.prefill(q, n, S, causal=bool(causal))
    ref = oracle_prefill(w, geom, kc, vc, q, n, causal=bool(causal), k_scale=ks, v_scale=vs)
    assert_close(got, ref, str(case))


def _check_query_partials(w, ws, q_len, m1, l1, ref):
    """As for decode: the live slots of every query row, re-referenced to the
    oracle's largest logit, sum to the oracle's l and combine to its output;
    their reference m lies within 8 ln 2 below the largest logit they saw. A
    row without keys has no live slot."""
    B, Hq = w.num_seqs, w.num_q_heads
    for b in range(B):
        for i in range(q_len):
            for h in range(Hq):
                l = ws[b, i, h, :, -1].astype(np.float64)
                m = ws[b, i, h, :, -2].astype(np.float64)
                marks = np.nonzero(l < 0)[0]
                stop = marks[0] if marks.size else l.size
                live = (l > 0) & (np.arange(l.size) < stop)
                if w.seq_lens[b] == 0:
                    continue
                if l1[b, i, h] == 0:
                    assert not live.any()
                    continue
                M, mo = m[live].max(), m1[b, i, h]
                tol = 1e-5 * max(1.0, abs(mo))
                assert mo - 8 * np.log(2.0) - tol <= M <= mo + tol
                wgt = l[live] * np.exp(m[live] - mo)
                assert abs(wgt.sum() - l1[b, i, h]) <= 1e-2 * l1[b, i, h]
                comb = (wgt[:, None] * ws[b, i, h, live, :-2]).sum(axis=0) / wgt.sum()
                assert np.max(np.abs(comb - ref[b, i, h])) <= 1e-2


@pytest.mark.parametrize("causal,window", [(1, 0), (1, 45), (0, 0)])
def test_prefill_partials(causal, window):
    w, geom, d, kc, vc, ks, vs = _setup("bf16", (3, 60, 300, 1000), 16, 2, 128, 16, window, 21)
    n = 6
    q = workloads.query_block(w, n, seed=4)
    got, ws = d.prefill(q, n, 9, causal=bool(causal), return_ws=True)
    ref, m1, l1 = oracle_prefill(w, geom, kc, vc, q, n, causal=bool(causal), return_state=True)
    assert_close(got, ref, "partials")
    _check_query_partials(w, ws, n, m1, l1, ref)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_one_token_block_is_decode(fmt):
    """q_len 1 runs the decode computation: bit-identical outputs."""
    D = 512 if fmt == "nvfp4" else 128
    w, geom, d, kc, vc, ks, vs = _setup(fmt, (1, 40, 333, 0), 8, 2, D, 16, 0, 31)
    for S in (1, 4):
        a = d.prefill(w.q_bits, 1, S, causal=True)
        b = d.prefill(w.q_bits, 1, S, causal=False)
        c = d.decode_single(S)
        assert np.array_equal(a[:, 0], c) and np.array_equal(b[:, 0], c)


def test_tokens_before_the_sequence_get_zeros():
    w, geom, d, kc, vc, ks, vs = _setup("bf16", (1, 3, 20), 4, 2, 64, 16, 0, 5)
    n = 6
    q = workloads.query_block(w, n, seed=9)
    for S in (1, 3):
        got = d.prefill(q, n, S)
        assert np.all(got[0, :5] == 0) and np.all(got[1, :3] == 0)
        assert np.all(np.isfinite(got))
        assert_close(got, oracle_prefill(w, geom, kc, vc, q, n), f"S={S}")


def test_strided_query_rows():
    w, geom, d, kc, vc, ks, vs = _setup("bf16", (100, 513, 40), 16, 4, 128, 16, 0, 6)
    n = 3
    q = workloads.query_block(w, n, seed=2)
    row = 16 * 128
    tok, seq = row + 64, 3 * (row + 64) + 32
    qp = np.full(3 * seq, 0x7FC0, np.uint16)                  # NaN padding must not be read
    for b in range(3):
        for i in range(n):
            qp[b * seq + i * tok: b * seq + i * tok + row] = q[b, i].reshape(-1)
    ref = oracle_prefill(w, geom, kc, vc, q, n)
    for S in (1, 5):
        assert_close(d.prefill(qp, n, S, q_stride=seq, q_token_stride=tok), ref, f"S={S}")


def test_deterministic_and_split_invariant():
    w, geom, d, kc, vc, ks, vs = _setup("bf16", (100, 513, 40), 16, 4, 128, 16, 0, 7)
    n = 4
    q = workloads.query_block(w, n, seed=3)
    ref = oracle_prefill(w, geom, kc, vc, q, n)
    a = d.prefill(q, n, 5)
    assert np.array_equal(a, d.prefill(q, n, 5))
    for S in (1, 2, 33, 200):
        assert_close(d.prefill(q, n, S), ref, f"S={S}")


@pytest.mark.parametrize("name,q_len", [("llama8b", 4), ("llama8b", 8), ("fp8", 2),
                                        ("nvfp4", 2)])
def test_full_size_speculative_verify(name, q_len):
    """Full-size workloads with a q_len-token verify block per sequence, at
    the split count the heuristic picks; every sequence against the oracle."""
    w, geom, ks, vs, kc, vc, _ = full_size_reference(name)
    print(f"[{name} q_len={q_len}] B={w.num_seqs} T={w.num_tokens}", flush=True)
    d = DeviceKV(w, geom, ks, vs)
    S = pkd.paged_prefill_num_splits(w.num_seqs, q_len, w.num_q_heads, w.num_kv_heads,
                                     w.max_blocks_per_seq, w.block_size, True,
                                     w.sliding_window, _num_cus())
    q = workloads.query_block(w, q_len, seed=1)
    got = d.prefill(q, q_len, S)
    ref = oracle_prefill(w, geom, kc, vc, q, q_len, k_scale=ks, v_scale=vs)
    err = assert_close(got, ref, name)
    print(f"[{name} q_len={q_len}] num_splits={S} all {w.num_seqs} seqs max_abs_err={err:.3e}",
          flush=True)
    del d
    torch.cuda.empty_cache()
