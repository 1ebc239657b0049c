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
from gpu_cases import (DeviceKV, assert_close, dev, geometry, i32_to_dev, oracle_pools,
                       u16_to_dev)

pytestmark = pytest.mark.gpu


def _tensor(rows, layout, Lmax, fill, dtype):
    """Per-sequence rows [L, Hkv, D] laid into (b, l, h, d) or (b, h, l, d)."""
    B = len(rows)
    Hkv, D = rows[0].shape[1], rows[0].shape[2]
    t = np.full((B, Lmax, Hkv, D), fill, dtype)
    for b, r in enumerate(rows):
        t[b, :len(r)] = r
    if layout == "bhld":
        t = np.ascontiguousarray(t.transpose(0, 2, 1, 3))
    return t, pkd.layout_strides(layout, B, Lmax, Hkv, D)


def _seq_rows(w, bits):
    out, start = [], 0
    for L in w.seq_lens:
        out.append(bits[start:start + int(L)])
        start += int(L)
    return out


class Contig:
    """A workload's K/V as contiguous device tensors (BF16, or FP8 codes from
    the oracle's encoder: inputs, read the same by both sides)."""

    def __init__(self, w, layout, fmt="bf16", k_scale=1.0, v_scale=1.0, pad=3, Lmax=None):
        self.w, self.fmt = w, fmt
        self.Lmax = int(max(1, w.seq_lens.max(initial=1))) + pad if Lmax is None else Lmax
        kr, vr = _seq_rows(w, w.k_bits), _seq_rows(w, w.v_bits)
        if fmt == "fp8":
            kr = [oracle.e4m3_encode(oracle.bf16_to_f64(r).astype(np.float32), k_scale) for r in kr]
            vr = [oracle.e4m3_encode(oracle.bf16_to_f64(r).astype(np.float32), v_scale) for r in vr]
            fill, dt = 0x7F, np.uint8                          # NaN codes in the padding
        else:
            fill, dt = 0x7FC0, np.uint16
        self.k_np, self.ks = _tensor(kr, layout, self.Lmax, fill, dt)
        self.v_np, self.vs = _tensor(vr, layout, self.Lmax, fill, dt)
        if fmt == "fp8":
            self.k = torch.from_numpy(self.k_np.reshape(-1)).to(dev())
            self.v = torch.from_numpy(self.v_np.reshape(-1)).to(dev())
        else:
            self.k = u16_to_dev(self.k_np.reshape(-1))
            self.v = u16_to_dev(self.v_np.reshape(-1))
        self.k_scale, self.v_scale = k_scale, v_scale

    def run(self, q, q_len, num_splits, causal=True, window=None, q_strides=None,
            o_layout="blhd", o_pad=0):
        w = self.w
        B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
        window = w.sliding_window if window is None else window
        if q_strides is None:
            q_strides = (q_len * Hq * D, Hq * D, D)
        # output: (b, i, h, d) or (b, h, i, d), each head row padded by o_pad elements
        row = D + o_pad
        if o_layout == "blhd":
            os_ = (q_len * Hq * row, Hq * row, row)
        else:
            os_ = (Hq * q_len * row, row, q_len * row)
        out = torch.full((B * q_len * Hq * row,), float("nan"), dtype=torch.bfloat16, device=dev())
        ws = None
        if num_splits > 1:
            ws = torch.full((pkd.paged_decode_workspace_bytes(B, Hq * q_len, D, num_splits) // 4,),
                            float("nan"), dtype=torch.float32, device=dev())
        qd = u16_to_dev(np.asarray(q).reshape(-1))
        lens = i32_to_dev(w.seq_lens)
        args = (qd, self.k, self.v, out, lens, B, q_len, self.Lmax, Hq, Hkv, D, float(w.scale))
        kw = dict(causal=causal, sliding_window=window, workspace=ws, num_splits=num_splits)
        if self.fmt == "fp8":
            pkd.contig_kv_attn_fp8(*args, self.k_scale, self.v_scale, q_strides, self.ks, self.vs,
                                   os_, **kw)
        else:
            pkd.contig_kv_attn_bf16(*args, q_strides, self.ks, self.vs, os_, **kw)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy().astype(np.float64)
        idx = (np.arange(B)[:, None, None, None] * os_[0] + np.arange(q_len)[None, :, None, None] * os_[1]
               + np.arange(Hq)[None, None, :, None] * os_[2] + np.arange(D)[None, None, None, :])
        return o[idx]

    def oracle(self, q, q_len, causal=True, window=None, q_strides=None, seqs=None):
        w = self.w
        Hq, D = w.num_q_heads, w.head_dim
        if q_strides is None:
            q_strides = (q_len * Hq * D, Hq * D, D)
        return oracle.contiguous_attention(
            self.fmt, q, self.k_np, self.v_np, w.seq_lens, Hq, w.num_kv_heads, D, q_len, w.scale,
            q_strides, self.ks, self.vs, causal=causal,
            sliding_window=w.sliding_window if window is None else window,
            k_scale=self.k_scale, v_scale=self.v_scale, seqs=seqs)


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
    """B=32, lengths U[512, 4096], (b, h, l, d) K/V: sampled sequences
    against the oracle at the heuristic split count, and the whole batch bit
    for bit against the paged decode of the same rows."""
    w = workloads.make_workload("llama8b")
    S = pkd.paged_decode_num_splits(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                    w.max_blocks_per_seq, w.block_size, 0,
                                    torch.cuda.get_device_properties(0).multi_processor_count)
    c = Contig(w, "bhld", Lmax=w.max_blocks_per_seq * w.block_size)
    got = c.run(w.q_bits.reshape(w.num_seqs, 1, w.num_q_heads, w.head_dim), 1, S)
    order = np.argsort(w.seq_lens)
    seqs = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2])})
    ref = c.oracle(w.q_bits.reshape(w.num_seqs, 1, w.num_q_heads, w.head_dim), 1, seqs=seqs)
    err = assert_close(got[seqs], ref, "llama8b contiguous")
    d = DeviceKV(w, geometry(w))
    paged = d.prefill(w.q_bits.reshape(w.num_seqs, 1, w.num_q_heads, w.head_dim), 1, S)
    assert np.array_equal(paged, got)
    print(f"[llama8b contiguous] S={S} seqs={seqs} max_abs_err={err:.3e}", flush=True)
