"""GPU parity: the HIP library, called through the C ABI, against the CPU
oracle on the same seeded inputs.

Cache writes and the absmax must match bit for bit; attention outputs must lie
within atol = rtol = 1e-2 of the float64 oracle (the tolerance of the AstrAI
paged and contiguous decode tests, restated in the problem statement).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_splitk_amd as pkd
import workloads
from gpu_cases import (DeviceKV, POISON, alloc_pool, assert_close, dev, fp8_scales,
                       full_size_reference, geometry, gpu_absmax, i32_to_dev, oracle_decode,
                       oracle_pools, pool_to_np, u16_to_dev)

pytestmark = pytest.mark.gpu


def _num_cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _fp8_small_scales(w):
    k = oracle.bf16_absmax(w.k_bits) / np.float32(448.0)
    v = oracle.bf16_absmax(w.v_bits) / np.float32(448.0)
    return np.float32(k), np.float32(v)


# ------------------------------------------------------------------ cache writes

@pytest.mark.parametrize("fmt,pad", [("bf16", 0), ("fp8", 0), ("fp8", 48), ("nvfp4", 0),
                                     ("nvfp4", 32)])
def test_cache_write_bit_exact(fmt, pad):
    w = workloads.make_workload("tiny", lens=(17, 40, 5, 64), num_q_heads=8, num_kv_heads=2,
                                head_dim=128, kv_dtype=fmt, sigma=1.5, seed=11)
    w.slot_mapping[[3, 20]] = -1                    # skipped tokens
    if fmt == "fp8":
        geom = geometry(w, cache_stride=16 * 2 * 128 + pad)
        ks, vs = _fp8_small_scales(w)
    elif fmt == "nvfp4":
        data = 16 * 2 * 128 // 2 + pad
        geom = geometry(w, data_section_bytes=data, block_stride_bytes=data + 16 * 2 * 8 + pad)
        ks = vs = 1.0
    else:
        geom = geometry(w)
        ks = vs = 1.0
    d = DeviceKV(w, geom, ks, vs)
    kc, vc = oracle_pools(w, geom, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(pool_to_np(d.k, fmt), kc)
    assert np.array_equal(pool_to_np(d.v, fmt), vc)


@pytest.mark.parametrize("scale", [1.0, 0.37, 1.0 / 448.0, 3.0e-3, 0.0])
def test_fp8_encoder_exhaustive_over_bf16(scale):
    """Every BF16 pattern (NaN and inf included) through the FP8 cache write."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    D, Hkv, bs = 256, 1, 16
    T = bits.size // D
    key = bits.reshape(T, Hkv, D)
    val = key[::-1].copy()
    slots = np.arange(T, dtype=np.int32)[::-1].copy()
    geom = oracle.CacheGeometry("fp8", (T + bs - 1) // bs, bs, Hkv, D)
    kc, vc = oracle.new_cache(geom, 0), oracle.new_cache(geom, 0)
    oracle.reshape_and_cache(geom, key, val, kc, vc, slots, k_scale=scale, v_scale=scale)
    kd = torch.zeros(kc.size, dtype=torch.uint8, device=dev())
    vd = torch.zeros_like(kd)
    pkd.reshape_and_cache_fp8(u16_to_dev(key), u16_to_dev(val), kd, vd, i32_to_dev(slots), Hkv, D,
                              bs, scale, scale)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().numpy(), kc)
    assert np.array_equal(vd.cpu().numpy(), vc)


def test_nvfp4_encoder_over_all_bf16():
    """Every BF16 pattern but NaN (infinities and subnormals included),
    shuffled into groups of 16, through the NVFP4 cache write, K and V in
    different groupings. A NaN in a group is outside the format's contract
    (the oracle's group maximum becomes NaN)."""
    rng = np.random.default_rng(11)
    allbits = np.arange(65536, dtype=np.uint32)
    nan = ((allbits & 0x7F80) == 0x7F80) & ((allbits & 0x7F) != 0)
    keep = allbits[~nan]
    pad = rng.choice(keep, 65536 - keep.size)            # back to whole 256-value rows
    bits = rng.permutation(np.concatenate([keep, pad])).astype(np.uint16)
    D, Hkv, bs = 256, 1, 16
    T = bits.size // D
    key = bits.reshape(T, Hkv, D)
    val = rng.permutation(bits).reshape(T, Hkv, D)
    slots = rng.permutation(T).astype(np.int32)
    geom = oracle.CacheGeometry("nvfp4", (T + bs - 1) // bs, bs, Hkv, D)
    kc, vc = oracle.new_cache(geom, 0xAB), oracle.new_cache(geom, 0xAB)
    oracle.reshape_and_cache(geom, key, val, kc, vc, slots)
    kd = torch.full((kc.size,), 0xAB, dtype=torch.uint8, device=dev())
    vd = kd.clone()
    pkd.reshape_and_cache_nvfp4(u16_to_dev(key), u16_to_dev(val), kd, vd, i32_to_dev(slots), Hkv, D,
                                bs)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().numpy(), kc)
    assert np.array_equal(vd.cpu().numpy(), vc)


def test_nvfp4_encoder_ties_and_ranges():
    """Groups at exact E2M1 ties, saturating scales and a wide magnitude range."""
    rng = np.random.default_rng(5)
    G = 4096
    S = oracle.e4m3_decode(rng.integers(0x08, 0x70, G).astype(np.uint8))
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0, 0.5, 1.0, 3.0, 4.0, 0.1, 2.2,
                     5.9])
    x = (S[:, None] * rng.permutation(np.tile(ties, (G, 1)).T).T
         * np.where(rng.random((G, 16)) < 0.5, -1.0, 1.0))
    x[: G // 4] *= rng.uniform(0.5, 1.5, (G // 4, 1))          # off-grid groups
    x[G // 4: G // 2] = rng.standard_normal((G // 4, 16)) * np.exp(rng.uniform(-8, 8, (G // 4, 1)))
    bits = workloads.bf16_bits_from_f32(x.astype(np.float32))
    D, Hkv, bs = 512, 1, 16
    T = bits.size // D
    key = bits.reshape(T, Hkv, D)
    slots = rng.permutation(T).astype(np.int32)
    geom = oracle.CacheGeometry("nvfp4", (T + bs - 1) // bs, bs, Hkv, D)
    kc, vc = oracle.new_cache(geom, 0xAB), oracle.new_cache(geom, 0xAB)
    oracle.reshape_and_cache(geom, key, key, kc, vc, slots)
    kd = torch.full((kc.size,), 0xAB, dtype=torch.uint8, device=dev())
    vd = kd.clone()
    pkd.reshape_and_cache_nvfp4(u16_to_dev(key), u16_to_dev(key), kd, vd, i32_to_dev(slots), Hkv, D,
                                bs)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().numpy(), kc)


@pytest.mark.parametrize("n", [1, 7, 8, 1000, 65536 + 3, 3_000_001])
def test_absmax_bit_exact(n):
    rng = np.random.default_rng(n)
    x = workloads.bf16_bits_from_f32((rng.standard_normal(n) * 3).astype(np.float32))
    if n > 10:
        x[rng.integers(0, n, 5)] = 0x7FC0           # NaN is ignored
        x[n - 1] = workloads.bf16_bits_from_f32(np.array([-1000.0], np.float32))[0]  # in the tail
    assert np.float32(gpu_absmax(x)) == oracle.bf16_absmax(x)


def test_absmax_folds_into_existing_value():
    x = workloads.bf16_bits_from_f32(np.array([1.0, -2.0, 3.0, 0.5] * 64, np.float32))
    out = torch.tensor([10.0], dtype=torch.float32, device=dev())
    pkd.bf16_absmax(u16_to_dev(x), out)
    torch.cuda.synchronize()
    assert float(out.item()) == 10.0


# ------------------------------------------------------------------ decode, small cases

def _check_partials(w, geom, kc, vc, ws, ref, ks=1.0, vs=1.0):
    """Each used workspace slot is a softmax partial over some keys, its l
    taken against a reference m at most 8 ln 2 below the piece's largest
    logit. Together they must reproduce the oracle's one-piece state (largest
    logit, sum of exponentials, both re-referenced to the oracle's m) and,
    weighted as the combine weighs them, its output."""
    o1, m1, l1 = oracle.split_partials(geom, w.q_bits, kc, vc, w.block_tables, w.seq_lens,
                                       w.num_q_heads, w.scale, 1, w.max_blocks_per_seq,
                                       sliding_window=w.sliding_window, k_scale=ks, v_scale=vs)
    B, Hq = w.num_seqs, w.num_q_heads
    for b in range(B):
        for h in range(Hq):
            l = ws[b, h, :, -1].astype(np.float64)
            m = ws[b, h, :, -2].astype(np.float64)
            marks = np.nonzero(l < 0)[0]
            stop = marks[0] if marks.size else l.size     # end marker: later slots ignored
            live = (l > 0) & (np.arange(l.size) < stop)
            if w.seq_lens[b] == 0:
                continue
            assert live.any()
            M, mo = m[live].max(), m1[b, h, 0]
            tol = 1e-5 * max(1.0, abs(mo))
            assert mo - 8 * np.log(2.0) - tol <= M <= mo + tol
            wgt = l[live] * np.exp(m[live] - mo)
            assert abs(wgt.sum() - l1[b, h, 0]) <= 1e-2 * l1[b, h, 0]
            comb = (wgt[:, None] * ws[b, h, live, :-2]).sum(axis=0) / wgt.sum()
            assert np.max(np.abs(comb - ref[b, h])) <= 1e-2


@pytest.mark.parametrize("S", [1, 3, 8])
def test_tiny_decode_and_partials(S):
    w = workloads.make_workload("tiny")
    geom = geometry(w)
    d = DeviceKV(w, geom)
    kc, vc = oracle_pools(w, geom)
    got, ws = d.decode(S, return_ws=True)
    ref = oracle_decode(w, geom, kc, vc)
    assert_close(got, ref, f"tiny S={S}")
    _check_partials(w, geom, kc, vc, ws, ref)


def test_partials_fp8_and_window():
    w = workloads.make_workload("tiny", lens=(1, 17, 300, 1000), num_q_heads=16, num_kv_heads=8,
                                head_dim=256, sliding_window=129, kv_dtype="fp8", seed=9)
    geom = geometry(w)
    ks, vs = _fp8_small_scales(w)
    d = DeviceKV(w, geom, ks, vs)
    kc, vc = oracle_pools(w, geom, ks, vs)
    got, ws = d.decode(5, return_ws=True)
    ref = oracle_decode(w, geom, kc, vc, ks, vs)
    assert_close(got, ref, "fp8 window partials")
    _check_partials(w, geom, kc, vc, ws, ref, ks, vs)


def test_stale_workspace_is_harmless():
    """The workspace may hold anything on entry (here NaN everywhere)."""
    w = workloads.make_workload("tiny", lens=(100, 513, 40, 0, 7), num_q_heads=16, num_kv_heads=4,
                                head_dim=128, seed=12)
    geom = geometry(w)
    d = DeviceKV(w, geom)
    kc, vc = oracle_pools(w, geom)
    ref = oracle_decode(w, geom, kc, vc)
    for S in (2, 9, 40):
        got = d.decode(S, ws_fill=float("nan"))
        assert_close(got, ref, f"stale workspace S={S}")


CASES = [
    # fmt, lens, Hq, Hkv, D, bs, window, S
    ("bf16", (1, 15, 16, 17, 100, 300), 8, 2, 128, 16, 0, 1),
    ("bf16", (1, 15, 16, 17, 100, 300), 8, 2, 128, 16, 0, 4),
    ("bf16", (33, 257, 1000), 32, 8, 128, 16, 0, 7),
    ("bf16", (5, 77, 130), 4, 4, 64, 32, 0, 2),
    ("bf16", (64, 200), 16, 1, 256, 64, 0, 3),
    ("bf16", (50, 180), 8, 1, 512, 16, 0, 2),
    ("bf16", (90, 400), 40, 2, 128, 16, 0, 3),          # 20 q heads per kv head: two chunks
    ("bf16", (90, 400, 17), 6, 2, 64, 16, 37, 3),       # sliding window, mid-page start
    ("bf16", (90, 400, 17), 6, 2, 64, 128, 100, 2),
    ("fp8", (1, 17, 300, 1000), 16, 8, 256, 16, 0, 3),
    ("fp8", (1, 17, 300, 1000), 16, 8, 256, 16, 129, 5),
    ("fp8", (40, 333), 4, 2, 64, 32, 0, 2),
    ("fp8", (40, 333), 8, 1, 128, 16, 60, 2),
    ("fp8", (40, 100), 16, 2, 512, 16, 0, 2),
    ("nvfp4", (1, 17, 300, 1000), 16, 2, 512, 16, 0, 3),
    ("nvfp4", (1, 17, 300, 700), 16, 2, 512, 16, 200, 4),
    ("nvfp4", (40, 333), 8, 2, 128, 16, 0, 2),
    ("nvfp4", (40, 333), 8, 2, 64, 32, 0, 2),
    ("nvfp4", (40, 200), 4, 2, 256, 64, 0, 2),
    ("fp8", (90, 400), 40, 2, 128, 16, 0, 3),           # two head chunks
    ("fp8", (5, 77, 530), 4, 4, 256, 256, 0, 2),
    ("fp8", (0, 1, 2, 700), 16, 8, 256, 16, 0, 4),      # empty, one and two keys
    ("fp8", (33, 600), 8, 2, 512, 32, 300, 3),
    ("nvfp4", (90, 400, 17), 6, 2, 64, 16, 37, 3),
    ("nvfp4", (50, 300), 8, 8, 512, 128, 0, 1),
    ("nvfp4", (0, 1, 2, 700), 16, 2, 512, 16, 0, 4),
    ("nvfp4", (90, 400), 40, 2, 128, 16, 0, 5),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-D{c[4]}-G{c[2]//c[3]}-bs{c[5]}-W{c[6]}-S{c[7]}"
                                             for c in CASES])
def test_decode_matches_oracle(case):
    fmt, lens, Hq, Hkv, D, bs, window, S = case
    w = workloads.make_workload("tiny", lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                block_size=bs, sliding_window=window, kv_dtype=fmt, seed=D + S)
    geom = geometry(w)
    ks, vs = _fp8_small_scales(w) if fmt == "fp8" else (1.0, 1.0)
    d = DeviceKV(w, geom, ks, vs)
    kc, vc = oracle_pools(w, geom, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(pool_to_np(d.k, fmt), kc)          # both sides read the same bytes
    got = d.decode(S)
    ref = oracle_decode(w, geom, kc, vc, ks, vs)
    assert_close(got, ref, str(case))


def test_empty_and_single_key_sequences():
    w = workloads.make_workload("tiny", lens=(0, 1, 0, 1), num_q_heads=8, num_kv_heads=2,
                                head_dim=128, seed=3)
    geom = geometry(w)
    d = DeviceKV(w, geom)
    for S in (1, 2, 5):
        got = d.decode(S)
        assert np.all(got[[0, 2]] == 0)
        # one key: softmax weight exactly 1, the output is its V row, bit for bit
        V = oracle.bf16_to_f64(w.v_bits)                     # tokens: seq 1, seq 3
        for i, b in enumerate((1, 3)):
            for h in range(8):
                assert np.array_equal(got[b, h], V[i, h // 4])


def test_zero_query_gives_mean_of_values():
    w = workloads.make_workload("tiny", lens=(37, 200), num_q_heads=4, num_kv_heads=2,
                                head_dim=64, seed=4)
    q0 = np.zeros_like(w.q_bits)
    geom = geometry(w)
    d = DeviceKV(w, geom)
    got = d.decode(3, q_bits=q0)
    kc, vc = oracle_pools(w, geom)
    ref = oracle_decode(w, geom, kc, vc, q_bits=q0)
    assert_close(got, ref, "q = 0")


def test_q_stride_and_split_invariance():
    w = workloads.make_workload("tiny", lens=(100, 513, 40), num_q_heads=16, num_kv_heads=4,
                                head_dim=128, seed=6)
    geom = geometry(w)
    d = DeviceKV(w, geom)
    stride = 16 * 128 + 64
    qp = np.full((3, stride), 0x7FC0, np.uint16)              # NaN padding must not be read
    qp[:, :16 * 128] = w.q_bits.reshape(3, -1)
    kc, vc = oracle_pools(w, geom)
    ref = oracle_decode(w, geom, kc, vc)
    outs = [d.decode(S, q_bits=qp, q_stride=stride) for S in (1, 2, 9, 33, 200)]
    for o in outs:
        assert_close(o, ref, "q_stride / splits")


def test_deterministic():
    w = workloads.make_workload("tiny", lens=(100, 513, 40), num_q_heads=16, num_kv_heads=4,
                                head_dim=128, seed=7)
    d = DeviceKV(w, geometry(w))
    a = d.decode(5)
    b = d.decode(5)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ full-size workloads

def _full_size(name):
    """The full-size workload in the launch configuration the bench times
    (the library's split count): the pools written by the library equal the
    oracle's byte for byte (every page, the unwritten bytes of partial last
    pages included), and every sequence's output matches the oracle."""
    w, geom, ks, vs, kc, vc, ref = full_size_reference(name)
    fmt = w.kv_dtype
    print(f"[{name}] B={w.num_seqs} T={w.num_tokens} fmt={fmt}", flush=True)
    d = DeviceKV(w, geom, ks, vs)
    assert np.array_equal(pool_to_np(d.k, fmt), kc) and np.array_equal(pool_to_np(d.v, fmt), vc)
    S = pkd.paged_decode_num_splits(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                    w.max_blocks_per_seq, w.block_size, w.sliding_window,
                                    _num_cus())
    got = d.decode(S)
    err = assert_close(got, ref, name)
    print(f"[{name}] num_splits={S} all {w.num_seqs} seqs max_abs_err={err:.3e}", flush=True)
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["llama8b", "fp8", "nvfp4"])
def test_full_size_batched(name):
    _full_size(name)


@pytest.mark.parametrize("name", ["b1_1k", "b1_4k", "b1_8k", "b1_16k", "b1_32k"])
def test_full_size_b1_long_context(name):
    _full_size(name)


# ------------------------------------------------------------------ whole-decode call

SINGLE_CASES = [CASES[i] for i in (1, 2, 6, 7, 9, 10, 13, 14, 15, 17, 19, 21, 23, 25)]


@pytest.mark.parametrize("case", SINGLE_CASES,
                         ids=[f"{c[0]}-D{c[4]}-G{c[2]//c[3]}-bs{c[5]}-W{c[6]}" for c in SINGLE_CASES])
def test_whole_decode_matches_oracle(case):
    """One wave per row (S=1, the non-split decode) and the split-K pass plus
    the combine behind the one call (S > 1)."""
    fmt, lens, Hq, Hkv, D, bs, window, S = case
    w = workloads.make_workload("tiny", lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                block_size=bs, sliding_window=window, kv_dtype=fmt, seed=D + S)
    geom = geometry(w)
    ks, vs = _fp8_small_scales(w) if fmt == "fp8" else (1.0, 1.0)
    d = DeviceKV(w, geom, ks, vs)
    kc, vc = oracle_pools(w, geom, ks, vs)
    ref = oracle_decode(w, geom, kc, vc, ks, vs)
    for n_splits in (1, 2, S, 40):
        assert_close(d.decode_single(n_splits), ref, f"{case} whole decode S={n_splits}")


def test_whole_decode_empty_and_single_key():
    w = workloads.make_workload("tiny", lens=(0, 1, 0, 1, 300), num_q_heads=8, num_kv_heads=2,
                                head_dim=128, seed=3)
    geom = geometry(w)
    d = DeviceKV(w, geom)
    V = oracle.bf16_to_f64(w.v_bits)
    for S in (1, 3, 17, 33):
        got = d.decode_single(S)
        assert np.all(got[[0, 2]] == 0)
        for i, b in enumerate((1, 3)):
            for h in range(8):
                assert np.array_equal(got[b, h], V[i, h // 4])


def test_whole_decode_graph_replay():
    """Captured once, replayed with eager work in between: every replay gives
    the eager output, for the non-split form and the two-launch form."""
    w = workloads.make_workload("tiny", lens=(100, 513, 40, 7, 1200), num_q_heads=32,
                                num_kv_heads=8, head_dim=128, seed=14)
    d = DeviceKV(w, geometry(w))
    B, Hq, D = w.num_seqs, w.num_q_heads, w.head_dim
    q = u16_to_dev(w.q_bits.reshape(-1))
    bt, lens = i32_to_dev(w.block_tables), i32_to_dev(w.seq_lens)
    for S in (1, 9):
        eager = d.decode_single(S)
        ws = torch.empty(pkd.paged_decode_workspace_bytes(B, Hq, D, S) // 4, dtype=torch.float32,
                         device=dev())
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev())
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                pkd.paged_decode_attn_bf16(q, d.k, d.v, out, bt, lens, w.max_blocks_per_seq, B,
                                           Hq, w.num_kv_heads, D, w.block_size, float(w.scale),
                                           Hq * D, 0, ws, S)
        torch.cuda.synchronize()
        for rep in range(3):
            out.fill_(float("nan"))
            ws.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            got = out.float().cpu().numpy().astype(np.float64)
            assert np.array_equal(got, eager), (S, rep)
            d.decode(3)                                      # eager work between replays
        del graph


SHORT_CASES = [
    # fmt, lens, Hq, Hkv, D, bs, window, one launch expected
    ("bf16", (128,), 32, 8, 128, 16, 0, True),              # one sequence, 8 tiles per row
    ("bf16", (0, 5, 190, 64, 17, 100), 32, 8, 128, 16, 0, True),
    ("fp8", (30, 150, 1), 16, 8, 256, 16, 0, True),
    ("bf16", (1, 500, 333), 8, 2, 64, 16, 100, True),       # the window bounds the rows
    ("bf16", (0, 5, 190, 64, 17, 100) * 8, 32, 8, 128, 16, 0, False),   # 384 rows: two launches
    ("bf16", (40, 250), 32, 8, 128, 16, 0, False),          # 16 tiles per row: two launches
]


@pytest.mark.parametrize("case", SHORT_CASES,
                         ids=[f"{c[0]}-B{len(c[1])}-D{c[4]}-W{c[6]}" for c in SHORT_CASES])
def test_whole_decode_short_rows(case):
    """Short rows (at most 12 tiles by the block-table width or the window),
    all resident at once: the whole-decode call runs the one-launch form
    whatever num_splits says, so its output is that of num_splits 1, bit for
    bit; otherwise the split pass and the combine. Both against the oracle."""
    fmt, lens, Hq, Hkv, D, bs, window, one = case
    w = workloads.make_workload("tiny", lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                block_size=bs, sliding_window=window, kv_dtype=fmt, seed=len(lens))
    geom = geometry(w)
    ks, vs = _fp8_small_scales(w) if fmt == "fp8" else (1.0, 1.0)
    d = DeviceKV(w, geom, ks, vs)
    kc, vc = oracle_pools(w, geom, ks, vs)
    ref = oracle_decode(w, geom, kc, vc, ks, vs)
    single = d.decode_single(1)
    assert_close(single, ref, f"{case} S=1")
    S = pkd.paged_decode_num_splits(w.num_seqs, Hq, Hkv, w.max_blocks_per_seq, bs, window,
                                    _num_cus())
    for n_splits in sorted({2, S}):
        got = d.decode_single(n_splits)
        assert_close(got, ref, f"{case} S={n_splits}")
        if one:
            assert np.array_equal(got, single), f"S={n_splits}: not the one-launch form"
        assert np.all(got[w.seq_lens == 0] == 0)


@pytest.mark.parametrize("name", ["llama8b", "b1_32k", "fp8", "nvfp4"])
def test_whole_decode_full_size(name):
    w, geom, ks, vs, kc, vc, ref = full_size_reference(name)
    d = DeviceKV(w, geom, ks, vs)
    S = pkd.paged_decode_num_splits(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                    w.max_blocks_per_seq, w.block_size, w.sliding_window,
                                    _num_cus())
    for n_splits in (1, S):
        got = d.decode_single(n_splits)
        err = assert_close(got, ref, f"{name} S={n_splits}")
        print(f"[{name}] whole decode num_splits={n_splits} all {w.num_seqs} seqs "
              f"max_abs_err={err:.3e}", flush=True)
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,B,S", [("bf16", 65, 3), ("bf16", 300, 9), ("fp8", 130, 5),
                                     ("nvfp4", 97, 4), ("bf16", 1000, 2)])
def test_many_sequences(fmt, B, S):
    """More than 64 sequences: the rows are found by a scan over the lengths
    in memory instead of per-lane registers. Lengths include zeros."""
    rng = np.random.default_rng(B)
    lens = rng.integers(0, 200, size=B)
    lens[rng.integers(0, B, size=max(1, B // 10))] = 0
    D = {"bf16": 128, "fp8": 256, "nvfp4": 512}[fmt]
    Hq, Hkv = {"bf16": (8, 2), "fp8": (16, 8), "nvfp4": (16, 2)}[fmt]
    w = workloads.make_workload("tiny", lens=tuple(int(x) for x in lens), num_q_heads=Hq,
                                num_kv_heads=Hkv, head_dim=D, kv_dtype=fmt, seed=B)
    geom = geometry(w)
    ks, vs = _fp8_small_scales(w) if fmt == "fp8" else (1.0, 1.0)
    d = DeviceKV(w, geom, ks, vs)
    kc, vc = oracle_pools(w, geom, ks, vs)
    ref = oracle_decode(w, geom, kc, vc, ks, vs)
    assert_close(d.decode(S), ref, f"{fmt} B={B} split-K S={S}")
    for n_splits in (1, S):
        got = d.decode_single(n_splits)
        assert_close(got, ref, f"{fmt} B={B} whole decode S={n_splits}")
        assert np.all(got[w.seq_lens == 0] == 0)


# ------------------------------------------------------------------ split-K with append

def _append_decode(w, geom, ks, vs, S):
    """Pools holding every token but each sequence's last; the append call
    writes the last ones and attends. Returns (output, device pools)."""
    last = w.last_token_index()
    keep = np.setdiff1d(np.arange(w.num_tokens), last[last >= 0])
    d = DeviceKV(w, geom, ks, vs, tokens=keep)
    B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    rows = np.zeros((B, Hkv * D), np.uint16)
    rows_v = np.zeros((B, Hkv * D), np.uint16)
    live = last >= 0
    rows[live] = w.k_bits[last[live]].reshape(-1, Hkv * D)
    rows_v[live] = w.v_bits[last[live]].reshape(-1, Hkv * D)
    key, val = u16_to_dev(rows.reshape(-1)), u16_to_dev(rows_v.reshape(-1))
    q = u16_to_dev(w.q_bits.reshape(-1))
    bt, lens = i32_to_dev(w.block_tables), i32_to_dev(w.seq_lens)
    ws = torch.full((pkd.paged_decode_workspace_bytes(B, Hq, D, S) // 4,), float("nan"),
                    dtype=torch.float32, device=dev())
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev())
    common = (q, key, val, d.k, d.v, ws, bt, lens, w.max_blocks_per_seq, Hq, Hkv, D, bs,
              float(w.scale), S)
    if geom.fmt == "bf16":
        pkd.paged_decode_attn_splitk_append_bf16(*common, Hq * D, B, w.sliding_window)
    elif geom.fmt == "fp8":
        pkd.paged_decode_attn_splitk_append_fp8(*common, ks, vs, Hq * D, geom.fp8_stride(), B,
                                                w.sliding_window)
    else:
        stride, data = geom.nvfp4_sections()
        pkd.paged_decode_attn_splitk_append_nvfp4(*common, Hq * D, stride, data, B,
                                                  w.sliding_window)
    pkd.paged_decode_attn_reduce(ws, out, lens, Hq, D, S, B)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), d


APPEND_CASES = [
    ("bf16", (1, 15, 16, 17, 100, 300), 8, 2, 128, 16, 0, 4),
    ("bf16", (33, 0, 257, 1000), 40, 2, 128, 16, 0, 7),      # two head chunks, an empty row
    ("bf16", (90, 400, 17), 6, 2, 64, 32, 37, 3),
    ("bf16", (50, 180), 8, 1, 512, 16, 0, 2),                # head dim split over two waves
    ("bf16", (300, 700), 8, 2, 128, 16, 0, 1),               # one wave per row
    ("fp8", (1, 17, 300, 1000), 16, 8, 256, 16, 129, 5),
    ("fp8", (40, 100), 16, 2, 512, 16, 0, 2),
    ("nvfp4", (1, 17, 300, 700), 16, 2, 512, 16, 200, 4),
    ("nvfp4", (40, 333), 8, 2, 64, 32, 0, 2),
]


@pytest.mark.parametrize("case", APPEND_CASES,
                         ids=[f"{c[0]}-D{c[4]}-G{c[2]//c[3]}-bs{c[5]}-W{c[6]}-S{c[7]}"
                              for c in APPEND_CASES])
def test_split_k_append(case):
    """The appended tokens land bit for bit where reshape_and_cache puts them,
    and the output is bit for bit that of the separate write + split-K."""
    fmt, lens, Hq, Hkv, D, bs, window, S = case
    w = workloads.make_workload("tiny", lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                block_size=bs, sliding_window=window, kv_dtype=fmt, seed=D + S)
    geom = geometry(w)
    ks, vs = _fp8_small_scales(w) if fmt == "fp8" else (1.0, 1.0)
    got, d = _append_decode(w, geom, ks, vs, S)
    kc, vc = oracle_pools(w, geom, ks, vs)
    assert np.array_equal(pool_to_np(d.k, fmt), kc) and np.array_equal(pool_to_np(d.v, fmt), vc)
    ref = oracle_decode(w, geom, kc, vc, ks, vs)
    assert_close(got, ref, f"append {case}")
    full = DeviceKV(w, geom, ks, vs)
    assert np.array_equal(got, full.decode(S))


@pytest.mark.parametrize("name", ["llama8b", "b1_32k", "fp8", "nvfp4"])
def test_split_k_append_full_size(name):
    """The decode step the bench times: pools holding every token but each
    sequence's last, the append call writing those and attending. Pools and
    outputs of every sequence against the oracle's."""
    w, geom, ks, vs, kc, vc, ref = full_size_reference(name)
    S = pkd.paged_decode_num_splits(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                    w.max_blocks_per_seq, w.block_size, w.sliding_window,
                                    _num_cus())
    got, d = _append_decode(w, geom, ks, vs, S)
    fmt = w.kv_dtype
    assert np.array_equal(pool_to_np(d.k, fmt), kc) and np.array_equal(pool_to_np(d.v, fmt), vc)
    err = assert_close(got, ref, f"{name} append")
    print(f"[{name}] append num_splits={S} all {w.num_seqs} seqs max_abs_err={err:.3e}",
          flush=True)
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,pad", [("fp8", 48), ("fp8", 4096), ("nvfp4", 32), ("nvfp4", 256)])
def test_decode_padded_pages(fmt, pad):
    """Pages with room between them (and NVFP4 scale sections that do not
    follow the codes directly): the split-K pass, the whole-decode call and
    the append call all address them through the strides."""
    w = workloads.make_workload("tiny", lens=(30, 333, 1, 70), num_q_heads=8, num_kv_heads=2,
                                head_dim=128, kv_dtype=fmt, seed=21)
    rows = 16 * 2 * 128
    if fmt == "fp8":
        geom = geometry(w, cache_stride=rows + pad)
        ks, vs = _fp8_small_scales(w)
    else:
        geom = geometry(w, data_section_bytes=rows // 2 + pad,
                        block_stride_bytes=rows // 2 + pad + rows // 16 + pad)
        ks = vs = 1.0
    d = DeviceKV(w, geom, ks, vs)
    kc, vc = oracle_pools(w, geom, ks, vs)
    assert np.array_equal(pool_to_np(d.k, fmt), kc)
    ref = oracle_decode(w, geom, kc, vc, ks, vs)
    assert_close(d.decode(3), ref, f"{fmt} pad {pad} split-K")
    assert_close(d.decode_single(1), ref, f"{fmt} pad {pad} non-split")
    got, da = _append_decode(w, geom, ks, vs, 3)
    assert np.array_equal(pool_to_np(da.k, fmt), kc) and np.array_equal(pool_to_np(da.v, fmt), vc)
    assert_close(got, ref, f"{fmt} pad {pad} append")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_cache_write_from_strided_rows(fmt):
    """K and V as slices of a fused QKV row (key_stride, value_stride larger
    than a row): the bytes written are those of the packed rows."""
    w = workloads.make_workload("tiny", lens=(17, 40, 5), num_q_heads=8, num_kv_heads=2,
                                head_dim=64, kv_dtype=fmt, sigma=1.5, seed=12)
    geom = geometry(w)
    ks, vs = _fp8_small_scales(w) if fmt == "fp8" else (1.0, 1.0)
    Hq, Hkv, D, T = w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_tokens
    row = Hkv * D
    width = Hq * D + 2 * row + 8                    # q | k | v | padding, per token
    qkv = np.full((T, width), 0x7FC0, np.uint16)
    qkv[:, Hq * D:Hq * D + row] = w.k_bits.reshape(T, row)
    qkv[:, Hq * D + row:Hq * D + 2 * row] = w.v_bits.reshape(T, row)
    buf = u16_to_dev(qkv.reshape(-1))
    key, val = buf[Hq * D:], buf[Hq * D + row:]
    kd, vd = alloc_pool(geom, POISON[fmt]), alloc_pool(geom, POISON[fmt])
    slots = i32_to_dev(w.slot_mapping)
    if fmt == "bf16":
        pkd.reshape_and_cache_bf16(key, val, kd, vd, slots, Hkv, D, w.block_size, width, width)
    elif fmt == "fp8":
        pkd.reshape_and_cache_fp8(key, val, kd, vd, slots, Hkv, D, w.block_size, ks, vs,
                                  key_stride=width, value_stride=width)
    else:
        pkd.reshape_and_cache_nvfp4(key, val, kd, vd, slots, Hkv, D, w.block_size,
                                    key_stride=width, value_stride=width)
    torch.cuda.synchronize()
    kc, vc = oracle_pools(w, geom, ks, vs)
    assert np.array_equal(pool_to_np(kd, fmt), kc) and np.array_equal(pool_to_np(vd, fmt), vc)


def test_lengths_past_the_block_table_are_clamped():
    """A seq_len beyond what the sequence's block-table row holds reads no
    further than the row: the sequence attends the keys its pages hold."""
    w = workloads.make_workload("tiny", lens=(17, 64), num_q_heads=4, num_kv_heads=2,
                                head_dim=64, seed=21)
    assert w.max_blocks_per_seq * w.block_size == 64
    geom = geometry(w)
    d = DeviceKV(w, geom)
    kc, vc = oracle_pools(w, geom)
    ref = oracle_decode(w, geom, kc, vc)
    too_long = np.array([17, 5000], np.int32)
    for S in (1, 3):
        got = d.decode(S, seq_lens=too_long)
        assert_close(got, ref, f"clamped S={S}")
        assert_close(d.decode_single(S), ref, f"whole S={S}")


def test_append_skips_lengths_past_the_block_table():
    """The split-K append with a length beyond the sequence's block-table row
    writes nothing for that sequence (its stored keys stay), while a sequence
    within its row appends as usual. The appended rows of the long sequence
    are NaN patterns, so a write anywhere in its pages would show."""
    w = workloads.make_workload("tiny", lens=(17, 64), num_q_heads=4, num_kv_heads=2,
                                head_dim=64, seed=21)
    geom = geometry(w)
    d = DeviceKV(w, geom)
    kc, vc = oracle_pools(w, geom)
    ref = oracle_decode(w, geom, kc, vc)
    B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    last = w.last_token_index()
    rows_k = np.full((B, Hkv * D), POISON["bf16"], np.uint16)
    rows_v = np.full((B, Hkv * D), POISON["bf16"], np.uint16)
    rows_k[0] = w.k_bits[last[0]].reshape(-1)            # sequence 0 re-appends its last key
    rows_v[0] = w.v_bits[last[0]].reshape(-1)
    key, val = u16_to_dev(rows_k.reshape(-1)), u16_to_dev(rows_v.reshape(-1))
    q = u16_to_dev(w.q_bits.reshape(-1))
    bt = i32_to_dev(w.block_tables)
    lens = i32_to_dev(np.array([17, 5000], np.int32))
    for S in (1, 3):
        ws = torch.full((pkd.paged_decode_workspace_bytes(B, Hq, D, S) // 4,), float("nan"),
                        dtype=torch.float32, device=dev())
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev())
        pkd.paged_decode_attn_splitk_append_bf16(q, key, val, d.k, d.v, ws, bt, lens,
                                                 w.max_blocks_per_seq, Hq, Hkv, D, bs,
                                                 float(w.scale), S, Hq * D, B)
        pkd.paged_decode_attn_reduce(ws, out, lens, Hq, D, S, B)
        torch.cuda.synchronize()
        assert np.array_equal(pool_to_np(d.k, "bf16"), kc), f"K pool changed, S={S}"
        assert np.array_equal(pool_to_np(d.v, "bf16"), vc), f"V pool changed, S={S}"
        assert_close(out.float().cpu().numpy().astype(np.float64), ref, f"append clamped S={S}")
