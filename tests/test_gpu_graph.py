"""HIP-graph capture and replay of the decode step as a serving loop runs it
(the pages' graph-replay requirement: bit-exact outputs and KV-cache
coverage across replays).

One decode step (split-K pass with the append, then the combine) is
captured once over fixed device buffers. Each replay is fed the next
token's q / K / V rows and the advanced sequence lengths by plain copies
outside the graph, with unrelated eager library work in between. Every
replay must equal the eager step on the same inputs bit for bit and the
oracle within atol = rtol = 1e-2, and after the last replay the cache must
hold every appended token exactly as the oracle's cache write puts it.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_splitk_amd as pkd
import workloads
from gpu_cases import (DeviceKV, POISON, assert_close, dev, geometry, i32_to_dev,
                       oracle_pools, pool_to_np, u16_to_dev)

pytestmark = pytest.mark.gpu

STEPS = 6


class StepBuffers:
    """Fixed device buffers of one decode step and the step itself."""

    def __init__(self, d, w, num_splits):
        B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
        self.d, self.w, self.S = d, w, num_splits
        self.q = torch.zeros(B * Hq * D, dtype=torch.int16, device=dev())
        self.key = torch.zeros(B * Hkv * D, dtype=torch.int16, device=dev())
        self.val = torch.zeros_like(self.key)
        self.lens = torch.zeros(B, dtype=torch.int32, device=dev())
        self.bt = i32_to_dev(w.block_tables)
        self.ws = torch.zeros(pkd.paged_decode_workspace_bytes(B, Hq, D, num_splits) // 4,
                              dtype=torch.float32, device=dev())
        self.out = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=dev())

    def feed(self, q_bits, key_bits, val_bits, lens):
        self.q.copy_(torch.from_numpy(q_bits.reshape(-1).view(np.int16)))
        self.key.copy_(torch.from_numpy(key_bits.reshape(-1).view(np.int16)))
        self.val.copy_(torch.from_numpy(val_bits.reshape(-1).view(np.int16)))
        self.lens.copy_(torch.from_numpy(lens.astype(np.int32)))

    def step(self):
        d, w = self.d, self.w
        g = d.geom
        common = (self.q, self.key, self.val, d.k, d.v, self.ws, self.bt, self.lens,
                  w.max_blocks_per_seq, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                  float(w.scale), self.S)
        qs = w.num_q_heads * w.head_dim
        if g.fmt == "bf16":
            pkd.paged_decode_attn_splitk_append_bf16(*common, qs, w.num_seqs, w.sliding_window)
        elif g.fmt == "fp8":
            pkd.paged_decode_attn_splitk_append_fp8(*common, d.k_scale, d.v_scale, qs,
                                                    g.fp8_stride(), w.num_seqs, w.sliding_window)
        else:
            stride, data = g.nvfp4_sections()
            pkd.paged_decode_attn_splitk_append_nvfp4(*common, qs, stride, data, w.num_seqs,
                                                      w.sliding_window)
        pkd.paged_decode_attn_reduce(self.ws, self.out, self.lens, w.num_q_heads, w.head_dim,
                                     self.S, w.num_seqs)


def _setup(fmt, D, Hq, Hkv, window, seed):
    base = np.array([1, 16, 47, 300, 0, 1000])
    w = workloads.make_workload("tiny", lens=tuple(base + STEPS), num_q_heads=Hq, num_kv_heads=Hkv,
                                head_dim=D, kv_dtype=fmt, sliding_window=window, seed=seed)
    if fmt == "fp8":
        ks = np.float32(oracle.bf16_absmax(w.k_bits) / np.float32(448.0))
        vs = np.float32(oracle.bf16_absmax(w.v_bits) / np.float32(448.0))
    else:
        ks = vs = 1.0
    prefix = w.token_pos < base[w.token_seq]
    return w, base, ks, vs, prefix


def _step_rows(w, base, r):
    """q (drawn per step) and the K / V rows of the token each sequence
    appends at step r (position base + r)."""
    idx = np.array([np.nonzero((w.token_seq == b) & (w.token_pos == base[b] + r))[0][0]
                    for b in range(w.num_seqs)])
    q = workloads.bf16_bits_from_f32(np.random.default_rng([r, 99]).standard_normal(
        (w.num_seqs, w.num_q_heads, w.head_dim), dtype=np.float32))
    return q, w.k_bits[idx], w.v_bits[idx]


@pytest.mark.parametrize("fmt,D,Hq,Hkv,window,S", [
    ("bf16", 128, 32, 8, 0, 9),
    ("bf16", 64, 8, 2, 40, 3),
    ("fp8", 256, 16, 8, 0, 5),
    ("nvfp4", 512, 16, 2, 0, 4),
])
def test_decode_loop_graph_replay(fmt, D, Hq, Hkv, window, S):
    w, base, ks, vs, prefix = _setup(fmt, D, Hq, Hkv, window, seed=D + S)
    geom = geometry(w)
    tokens = np.nonzero(prefix)[0]
    graph_kv = DeviceKV(w, geom, ks, vs, tokens=tokens)
    eager_kv = DeviceKV(w, geom, ks, vs, tokens=tokens)
    gb = StepBuffers(graph_kv, w, S)
    eb = StepBuffers(eager_kv, w, S)
    other = DeviceKV(w, geom, ks, vs, tokens=tokens)     # eager work between replays

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            gb.step()
    torch.cuda.synchronize()

    for r in range(STEPS):
        q, kr, vr = _step_rows(w, base, r)
        lens = base + r + 1
        gb.feed(q, kr, vr, lens)
        gb.out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = gb.out.float().cpu().numpy().astype(np.float64)

        eb.feed(q, kr, vr, lens)
        eb.step()
        torch.cuda.synchronize()
        want = eb.out.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, want), f"replay {r} differs from the eager step"

        upto = w.token_pos < (base + r + 1)[w.token_seq]
        kc, vc = oracle.new_cache(geom, POISON[fmt]), oracle.new_cache(geom, POISON[fmt])
        oracle.reshape_and_cache(geom, w.k_bits[upto], w.v_bits[upto], kc, vc,
                                 w.slot_mapping[upto], k_scale=ks, v_scale=vs)
        ref = oracle.paged_decode_attention(geom, q, kc, vc, w.block_tables, lens.astype(np.int32),
                                            Hq, w.scale, sliding_window=window, k_scale=ks,
                                            v_scale=vs)
        assert_close(got, ref, f"{fmt} replay {r}")
        other.decode(2)                                    # unrelated eager library work

    # coverage: every appended token sits in the cache exactly as the oracle writes it
    kc, vc = oracle_pools(w, geom, ks, vs)
    assert np.array_equal(pool_to_np(graph_kv.k, fmt), kc)
    assert np.array_equal(pool_to_np(graph_kv.v, fmt), vc)
    del graph


def test_multi_token_and_contiguous_graph_replay():
    """The multi-token call and the contiguous-K/V call captured once and
    replayed on fresh query blocks: bit-identical to eager calls."""
    w = workloads.make_workload("tiny", lens=(1, 17, 300, 1000, 64), num_q_heads=32,
                                num_kv_heads=8, head_dim=128, seed=8)
    d = DeviceKV(w, geometry(w))
    B, Hq, Hkv, D, n, S = w.num_seqs, 32, 8, 128, 4, 5
    qbuf = torch.zeros(B * n * Hq * D, dtype=torch.int16, device=dev())
    lens = i32_to_dev(w.seq_lens)
    bt = i32_to_dev(w.block_tables)
    ws = torch.zeros(pkd.paged_decode_workspace_bytes(B, Hq * n, D, S) // 4, dtype=torch.float32,
                     device=dev())
    out = torch.zeros((B, n, Hq, D), dtype=torch.bfloat16, device=dev())
    # a (b, l, h, d) copy of the same rows for the contiguous call
    Lmax = w.max_blocks_per_seq * w.block_size
    kd = np.zeros((B, Lmax, Hkv, D), np.uint16)
    vd = np.zeros((B, Lmax, Hkv, D), np.uint16)
    kd[w.token_seq, w.token_pos] = w.k_bits
    vd[w.token_seq, w.token_pos] = w.v_bits
    kt, vt = u16_to_dev(kd.reshape(-1)), u16_to_dev(vd.reshape(-1))
    kvs = pkd.layout_strides("blhd", B, Lmax, Hkv, D)
    qs = (n * Hq * D, Hq * D, D)
    out2 = torch.zeros_like(out)
    ws2 = torch.zeros_like(ws)

    def calls(o, w_, o2, w2):
        pkd.paged_prefill_attn_bf16(qbuf, d.k, d.v, o, bt, lens, w.max_blocks_per_seq, B, n, Hq,
                                    Hkv, D, w.block_size, float(w.scale), workspace=w_,
                                    num_splits=S)
        pkd.contig_kv_attn_bf16(qbuf, kt, vt, o2, lens, B, n, Lmax, Hq, Hkv, D, float(w.scale),
                                qs, kvs, kvs, qs, workspace=w2, num_splits=S)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            calls(out, ws, out2, ws2)
    torch.cuda.synchronize()
    e1, e2 = torch.zeros_like(out), torch.zeros_like(out)
    ew1, ew2 = torch.zeros_like(ws), torch.zeros_like(ws)
    for r in range(4):
        qb = workloads.query_block(w, n, seed=40 + r)
        qbuf.copy_(torch.from_numpy(qb.reshape(-1).view(np.int16)))
        out.fill_(float("nan"))
        out2.fill_(float("nan"))
        graph.replay()
        calls(e1, ew1, e2, ew2)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), e1.view(torch.int16)), r
        assert torch.equal(out2.view(torch.int16), e2.view(torch.int16)), r
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), r   # paged twin
    del graph
