"""The whole BF16 decode on the library's static scratch
(paged_decode_attn_bf16_noalloc, for callers that cannot allocate) against
the same call with a caller workspace (paged_decode_attn_bf16) and against the
oracle: two calls in a row, the second on a smaller input, then the size
limit."""
import numpy as np
import pytest
import torch

import paged_kv_decode_splitk_amd as pkd
import workloads
from gpu_cases import (DeviceKV, assert_close, dev, geometry, i32_to_dev, oracle_decode,
                       oracle_pools, u16_to_dev)

pytestmark = pytest.mark.gpu


def _both(w, d, S):
    """(output of the no-alloc call, output of the call with a workspace)."""
    B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    q = u16_to_dev(w.q_bits.reshape(-1))
    bt, lens = i32_to_dev(w.block_tables), i32_to_dev(w.seq_lens)
    common = (q, d.k, d.v)
    tail = (bt, lens, w.max_blocks_per_seq, B, Hq, Hkv, D, bs, float(w.scale), Hq * D)
    out_s = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=dev())
    pkd.paged_decode_attn_bf16_noalloc(*common, out_s, *tail, sliding_window=w.sliding_window,
                                       num_splits=S)
    ws = torch.full((pkd.paged_decode_workspace_bytes(B, Hq, D, S) // 4,), float("nan"),
                    dtype=torch.float32, device=dev())
    out_w = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=dev())
    pkd.paged_decode_attn_bf16(*common, out_w, *tail, sliding_window=w.sliding_window,
                               workspace=ws, num_splits=S)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return f(out_s), f(out_w)


def test_noalloc_matches_workspace_call_twice():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # first call: a batch of 5 llama-shaped sequences (one empty), heuristic split
    big = workloads.make_workload("tiny", lens=(300, 1000, 0, 57, 2000), num_q_heads=32,
                                  num_kv_heads=8, head_dim=128, seed=31)
    # second call: a smaller input (2 sequences, GQA 2, head_dim 64) on the same scratch
    small = workloads.make_workload("tiny")
    for w in (big, small):
        geom = geometry(w)
        d = DeviceKV(w, geom)
        kc, vc = oracle_pools(w, geom)
        ref = oracle_decode(w, geom, kc, vc)
        S = pkd.paged_decode_num_splits(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                        w.max_blocks_per_seq, w.block_size, w.sliding_window, cus)
        assert S > 1
        need = pkd.paged_decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.head_dim, S)
        print(f"[noalloc] B={w.num_seqs} Hq={w.num_q_heads} D={w.head_dim} S={S} "
              f"scratch bytes={need}", flush=True)
        for n_splits in (S, 1, 3):
            got, want = _both(w, d, n_splits)
            assert np.array_equal(got, want), f"S={n_splits}"
            assert_close(got, ref, f"noalloc S={n_splits}")
        assert np.all(got[w.seq_lens == 0] == 0)


def test_noalloc_rejects_more_than_the_scratch():
    w = workloads.make_workload("tiny", lens=(40, 17), num_q_heads=32, num_kv_heads=8,
                                head_dim=128, seed=5)
    d = DeviceKV(w, geometry(w))
    # 2 x 32 rows x S slots x 130 floats > 16 MiB for S = 1024
    S = 1024
    assert pkd.paged_decode_workspace_bytes(2, 32, 128, S) > pkd.SCRATCH_BYTES
    out = torch.zeros((2, 32, 128), dtype=torch.bfloat16, device=dev())
    with pytest.raises(pkd.PkdError, match="static scratch"):
        pkd.paged_decode_attn_bf16_noalloc(u16_to_dev(w.q_bits.reshape(-1)), d.k, d.v, out,
                                           i32_to_dev(w.block_tables), i32_to_dev(w.seq_lens),
                                           w.max_blocks_per_seq, 2, 32, 8, 128, w.block_size,
                                           float(w.scale), 32 * 128, num_splits=S)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0          # nothing was enqueued
