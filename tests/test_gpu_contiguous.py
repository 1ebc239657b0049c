"""GPU parity of attention over contiguous K/V tensors (no block table),
called through the C ABI, against the CPU oracle on the same seeded inputs
(atol = rtol = 1e-2), and bit for bit against the paged call over a paged
cache holding the same rows."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_splitk_amd as pkd
import workloads
from gpu_cases import Contig, DeviceKV, assert_close, geometry

pytestmark = pytest.mark.gpu


CASES = [
    # fmt, layout, lens, q_len, Hq, Hkv, D, causal, window, S
    ("bf16", "blhd", (17, 40), 1, 4, 2, 64, 1, 0, 1),
    ("bf16", "bhld", (17, 40), 1, 4, 2, 64, 1, 0, 3),
    ("bf16", "bhld", (1, 15, 16, 17, 100, 300), 4, 32, 8, 128, 1, 0, 5),
    ("bf16", "blhd", (33, 257, 1000), 8, 32, 8, 128, 1, 0, 7),        # two chunks per wave
    ("bf16", "bhld", (0, 5, 77, 130), 6, 4, 4, 64, 1, 0, 2),
    ("bf16", "blhd", (64, 200), 3, 16, 1, 256, 0, 0, 3),
    ("bf16", "bhld", (50, 180), 2, 8, 1, 512, 1, 0, 2),                # split head dim
    ("bf16", "blhd", (90, 400, 17), 5, 6, 2, 64, 1, 37, 3),
    ("bf16", "bhld", (90, 400, 17), 1, 6, 2, 64, 0, 37, 1),
    ("fp8", "blhd", (1, 17, 300, 1000), 2, 16, 8, 256, 1, 0, 3),
    ("fp8", "bhld", (1, 17, 300, 1000), 1, 16, 8, 256, 1, 129, 5),
    ("fp8", "bhld", (40, 333), 4, 8, 1, 128, 1, 60, 1),
    ("fp8", "blhd", (40, 100), 2, 16, 2, 512, 1, 0, 2),
    # FP8 rows of 64 bytes: the split pass runs kv heads in groups of two
    ("fp8", "bhld", (5, 300, 0, 777, 64), 1, 16, 4, 64, 0, 0, 5),
    ("fp8", "blhd", (5, 300, 0, 777, 64), 1, 8, 8, 64, 0, 200, 9),
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"{c[0]}-{c[1]}-n{c[3]}-D{c[6]}-G{c[4] // c[5]}-{'c' if c[7] else 'nc'}-W{c[8]}-S{c[9]}"
    for c in CASES])
def test_contiguous_matches_oracle(case):
    fmt, layout, lens, n, Hq, Hkv, D, causal, window, S = case
    w = workloads.make_workload("tiny", lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                sliding_window=window, seed=D + n + S)
    ks, vs = (np.float32(oracle.bf16_absmax(w.k_bits) / np.float32(448.0)),
              np.float32(oracle.bf16_absmax(w.v_bits) / np.float32(448.0))) if fmt == "fp8" \
        else (1.0, 1.0)
    c = Contig(w, layout, fmt, ks, vs)
    q = workloads.query_block(w, n, seed=S)
    got = c.run(q, n, S, causal=bool(causal))
    ref = c.oracle(q, n, causal=bool(causal))
    assert_close(got, ref, str(case))


def test_strided_q_and_output_layouts():
    w = workloads.make_workload("tiny", lens=(100, 513, 40), num_q_heads=16, num_kv_heads=4,
                                head_dim=128, seed=6)
    c = Contig(w, "bhld", pad=20)
    n, Hq, D = 3, 16, 128
    q = workloads.query_block(w, n, seed=2)
    ref = c.oracle(q, n)
    # q as (b, h, i, d) with a padded head row
    qp = np.full((3, Hq, n, D + 8), 0x7FC0, np.uint16)
    qp[..., :D] = q.transpose(0, 2, 1, 3)
    qs = (Hq * n * (D + 8), D + 8, n * (D + 8))
    for S in (1, 6):
        for ol, pad in (("blhd", 0), ("bhld", 24)):
            got = c.run(qp, n, S, q_strides=qs, o_layout=ol, o_pad=pad)
            assert_close(got, ref, f"S={S} out={ol}")


@pytest.mark.parametrize("n,S", [(1, 1), (1, 7), (4, 5), (8, 3)])
def test_paged_twin_is_bit_identical(n, S):
    """The same rows behind a shuffled block table: identical outputs."""
    w = workloads.make_workload("tiny", lens=(1, 17, 300, 1000, 64), num_q_heads=32,
                                num_kv_heads=8, head_dim=128, seed=8)
    d = DeviceKV(w, geometry(w))
    # the same key capacity as the block table: the same split plan
    c = Contig(w, "blhd", Lmax=w.max_blocks_per_seq * w.block_size)
    q = workloads.query_block(w, n, seed=5)
    paged = d.prefill(q, n, S)
    contig = c.run(q, n, S)
    assert np.array_equal(paged, contig)


def test_full_size_llama8b_contiguous():
    """B=32, lengths U[512, 4096], (b, h, l, d) K/V: every sequence against
    the oracle at the heuristic split count, and the whole batch bit for bit
    against the paged decode of the same rows."""
    w = workloads.make_workload("llama8b")
    S = pkd.paged_decode_num_splits(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                    w.max_blocks_per_seq, w.block_size, 0,
                                    torch.cuda.get_device_properties(0).multi_processor_count)
    c = Contig(w, "bhld", Lmax=w.max_blocks_per_seq * w.block_size)
    got = c.run(w.q_bits.reshape(w.num_seqs, 1, w.num_q_heads, w.head_dim), 1, S)
    ref = c.oracle(w.q_bits.reshape(w.num_seqs, 1, w.num_q_heads, w.head_dim), 1)
    err = assert_close(got, ref, "llama8b contiguous")
    d = DeviceKV(w, geometry(w))
    paged = d.prefill(w.q_bits.reshape(w.num_seqs, 1, w.num_q_heads, w.head_dim), 1, S)
    assert np.array_equal(paged, got)
    print(f"[llama8b contiguous] S={S} all {w.num_seqs} seqs max_abs_err={err:.3e}", flush=True)
