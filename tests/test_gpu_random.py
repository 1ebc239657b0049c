"""Seeded random sweep of shapes through every attention entry point against
the oracle (atol = rtol = 1e-2): cache format, head_dim, GQA group, block
size, batch and length mix (empty, single-key, tile- and page-boundary
lengths), window, split count, query-block length and causality, and for
BF16 / FP8 the contiguous-K/V call in a random layout. Each case prints
its parameters before it runs."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_splitk_amd as pkd
import workloads
from gpu_cases import Contig, DeviceKV, assert_close, geometry, oracle_pools, oracle_prefill

pytestmark = pytest.mark.gpu

NUM_CASES = 40


def _draw(i):
    rng = np.random.default_rng([2026, i])
    fmt = ["bf16", "fp8", "nvfp4"][i % 3]
    D = int(rng.choice([64, 128, 256, 512]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 20]))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    B = int(rng.integers(1, 7))
    specials = [0, 1, 15, 16, 17, bs - 1, bs, bs + 1, 2 * bs]
    lens = [int(rng.choice(specials)) if rng.random() < 0.35 else int(rng.integers(1, 700))
            for _ in range(B)]
    if max(lens) == 0:
        lens[0] = 5
    window = 0 if rng.random() < 0.6 else int(rng.integers(1, 400))
    q_len = 1 if rng.random() < 0.4 else int(rng.integers(2, 11))
    causal = bool(rng.random() < 0.8)
    S = int(rng.choice([1, 2, 3, 7, 33]))
    layout = str(rng.choice(["blhd", "bhld"]))
    return dict(fmt=fmt, D=D, Hkv=Hkv, Hq=Hkv * G, bs=bs, lens=tuple(lens), window=window,
                q_len=q_len, causal=causal, S=S, layout=layout, seed=i)


@pytest.mark.parametrize("i", range(NUM_CASES))
def test_random_shape(i):
    c = _draw(i)
    print(f"[random {i}] {c}", flush=True)
    w = workloads.make_workload("tiny", lens=c["lens"], num_q_heads=c["Hq"],
                                num_kv_heads=c["Hkv"], head_dim=c["D"], block_size=c["bs"],
                                sliding_window=c["window"], kv_dtype=c["fmt"], seed=c["seed"])
    geom = geometry(w)
    if c["fmt"] == "fp8":
        ks = np.float32(oracle.bf16_absmax(w.k_bits) / np.float32(448.0))
        vs = np.float32(oracle.bf16_absmax(w.v_bits) / np.float32(448.0))
    else:
        ks = vs = 1.0
    d = DeviceKV(w, geom, ks, vs)
    kc, vc = oracle_pools(w, geom, ks, vs)
    n = c["q_len"]
    q = workloads.query_block(w, n, seed=c["seed"])
    ref = oracle_prefill(w, geom, kc, vc, q, n, causal=c["causal"], k_scale=ks, v_scale=vs)
    got = d.prefill(q, n, c["S"], causal=c["causal"])
    assert_close(got, ref, f"paged {c}")
    if n == 1:
        # the decode entry points on the same query
        q1 = np.ascontiguousarray(q[:, 0])
        assert_close(d.decode(c["S"], q_bits=q1)[:, None], ref, f"split-K decode {c}")
        assert_close(d.decode_single(c["S"], q_bits=q1)[:, None], ref, f"whole decode {c}")
    if c["fmt"] != "nvfp4":
        ct = Contig(w, c["layout"], c["fmt"], ks, vs)
        got_c = ct.run(q, n, c["S"], causal=c["causal"])
        assert_close(got_c, ct.oracle(q, n, causal=c["causal"]), f"contiguous {c}")
    del d
    torch.cuda.empty_cache()
