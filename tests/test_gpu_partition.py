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


# NVFP4 batches whose kv heads share cache lines (scale rows of head_dim/16
# bytes, code rows under 128 bytes): the split-K pass runs the heads of a
# group as workgroups of one partition unit, 8 apart in the grid. Every head
# of every sequence is compared, in lengths-in-registers and from-memory
# batches, with and without a window.
GROUP_CASES = [
    # B, Hq, Hkv, D, lo, hi, window, seed
    (24, 16, 8, 128, 100, 2500, 0, 5),      # groups of 8 heads
    (70, 8, 4, 64, 50, 1200, 0, 6),         # groups of 4, lengths from memory
    (12, 16, 2, 512, 300, 4000, 700, 7),    # groups of 2, sliding window
    (16, 12, 6, 256, 1, 900, 0, 8),         # 6 heads: groups of 2
    (5, 40, 2, 128, 10, 900, 0, 9),         # G = 20: two column chunks per kv head
]


@pytest.mark.parametrize("B,Hq,Hkv,D,lo,hi,window,seed", GROUP_CASES)
def test_nvfp4_head_groups(B, Hq, Hkv, D, lo, hi, window, seed):
    lens = tuple(int(x) for x in np.random.default_rng(seed).integers(lo, hi, B, endpoint=True))
    print(f"[head groups] nvfp4 B={B} Hq={Hq} Hkv={Hkv} D={D} lens U[{lo},{hi}] W={window} "
          f"seed={seed}", flush=True)
    w = workloads.make_workload("nvfp4", lens=lens, num_q_heads=Hq, num_kv_heads=Hkv,
                                head_dim=D, sliding_window=window, seed=200 + seed)
    geom = geometry(w)
    d = DeviceKV(w, geom)
    kc, vc = oracle_pools(w, geom)
    ref = oracle_decode(w, geom, kc, vc)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    import paged_kv_decode_splitk_amd as pkd
    S = pkd.paged_decode_num_splits(B, Hq, Hkv, w.max_blocks_per_seq, w.block_size, window, cus)
    for n_splits in (S, 5):
        assert_close(d.decode(n_splits), ref, f"nvfp4 head groups S={n_splits}")
    del d
    torch.cuda.empty_cache()


def test_fp8_head_groups():
    """FP8 rows of head_dim 64 are 64 bytes: two kv heads share each line, and
    the split pass groups them in pairs (lengths in registers and from memory)."""
    import oracle
    import paged_kv_decode_splitk_amd as pkd
    for B, seed in ((24, 11), (80, 12)):
        lens = tuple(int(x) for x in np.random.default_rng(seed).integers(0, 1500, B))
        print(f"[head groups] fp8 B={B} Hkv=4 D=64 seed={seed}", flush=True)
        w = workloads.make_workload("fp8", lens=lens, num_q_heads=16, num_kv_heads=4,
                                    head_dim=64, sliding_window=0, seed=300 + seed)
        ks = np.float32(oracle.bf16_absmax(w.k_bits) / np.float32(448.0))
        vs = np.float32(oracle.bf16_absmax(w.v_bits) / np.float32(448.0))
        geom = geometry(w)
        d = DeviceKV(w, geom, ks, vs)
        kc, vc = oracle_pools(w, geom, ks, vs)
        ref = oracle_decode(w, geom, kc, vc, ks, vs)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        S = pkd.paged_decode_num_splits(B, 16, 4, w.max_blocks_per_seq, w.block_size, 0, cus)
        for n_splits in (S, 3):
            assert_close(d.decode(n_splits), ref, f"fp8 head groups B={B} S={n_splits}")
        del d
        torch.cuda.empty_cache()
