"""Batches shaped for the start-up positions of the stream partition.

The split-K pass lays each row of 16-key tiles behind up to three empty
positions, taken from the slack left when the per-wave tile count is rounded
up. The lengths below (seeded U[lo, hi] draws) were chosen so that on MI355X
(1,024 resident waves or workgroups for these calls) the count comes from the
rounding, not from the split-count floor, and the slack leaves two or three
positions per row: waves then hold ranges that end inside a row's positions,
rows start mid-wave, and slots count from the wave holding a row's first tile.
Batches of at most 64 sequences find rows from per-lane registers, larger ones
from memory; the 16-token causal block runs the shared-tile kernel. Every
output is compared with the oracle (atol = rtol = 1e-2). On another part the
same calls still run and are checked, with whatever slack it has."""
import numpy as np
import pytest
import torch

import workloads
from gpu_cases import DeviceKV, assert_close, geometry, oracle_decode, oracle_pools, oracle_prefill

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, lo, hi, seed, q_len
    (40, 32, 8, 200, 1500, 3, 1),       # lengths in registers
    (90, 8, 2, 200, 3000, 0, 1),        # lengths read from memory
    (90, 16, 4, 200, 2000, 0, 1),
    (40, 32, 8, 200, 1500, 3, 16),      # 64 query columns per kv head: waves share the tiles
]


@pytest.mark.parametrize("B,Hq,Hkv,lo,hi,seed,q_len", CASES)
def test_partition_start_up_positions(B, Hq, Hkv, lo, hi, seed, q_len):
    lens = tuple(int(x) for x in np.random.default_rng(seed).integers(lo, hi, B, endpoint=True))
    print(f"[partition] B={B} Hq={Hq} Hkv={Hkv} lens U[{lo},{hi}] seed={seed} q_len={q_len}",
          flush=True)
    w = workloads.make_workload("llama8b", lens=lens, num_q_heads=Hq, num_kv_heads=Hkv,
                                seed=100 + seed)
    geom = geometry(w)
    d = DeviceKV(w, geom)
    kc, vc = oracle_pools(w, geom)
    S = 17
    if q_len == 1:
        ref = oracle_decode(w, geom, kc, vc)
        assert_close(d.decode(S), ref, f"split-K decode B={B}")
    else:
        q = workloads.query_block(w, q_len, seed=seed)
        ref = oracle_prefill(w, geom, kc, vc, q, q_len, causal=True)
        assert_close(d.prefill(q, q_len, S, causal=True), ref, f"query block B={B}")
    del d
    torch.cuda.empty_cache()
