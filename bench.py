"""Benchmark of one paged decode step on one MI355X.

A step is the whole decode path for one attention layer over one batch: the
new token's K/V go into the cache, the split-KV pass runs, then the combine.
The headline step does it in two launches (the split-K pass that appends the
new token itself, then the combine); the same step with a separate
reshape_and_cache launch, and the non-split decode (one wave per row), are
timed beside it. Inputs are seeded
synthetic tensors already resident in HBM. Steps rotate over several layers'
KV pools whose total size is several times the 256 MB Infinity Cache, so
every step reads its KV from HBM, as the layers of a model do. The timed loop
replays a HIP graph of one step per layer.

Prints ONE JSON line: KV-read GB/s and us/step on the Llama-3-8B-shaped batch
(B=32), the B=1 32K-context figures beside it, the roofline of the step's
dominant kernel (back-to-back launches timed with HIP events on their
stream), and the float64 CPU oracle timed on the host. Beside them: a causal
query block of q_len tokens per sequence (speculative verify) over the same
batch, through the multi-token call (--verify workload:q_len), and the same
decode over contiguous K/V tensors (--contig workload:layout).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--extra NAME ...]
  python bench.py --verify-only --verify llama8b:4   # the multi-token call alone
  python bench.py --copy-calibration      # plain copy of known size (for rocprof counters)
  python bench.py --counter-run --workload NAME   # the split-K append call alone (rocprof counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV-read HBM GB/s (% of peak) + us/decode step, B=32 and B=1@32K ctx"
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20
DESCRIPTIONS = {
    "llama8b": "Llama-3-8B-shaped BF16 decode: B=32, 32 q / 8 kv heads, head_dim 128, block 16, "
               "seq_lens U[512, 4096], shuffled page pool",
    "b1_32k": "B=1 BF16 decode at 32K context: 32 q / 8 kv heads, head_dim 128, block 16",
    "b1_16k": "B=1 BF16 decode at 16K context: 32 q / 8 kv heads, head_dim 128, block 16",
    "b1_8k": "B=1 BF16 decode at 8K context: 32 q / 8 kv heads, head_dim 128, block 16",
    "b1_4k": "B=1 BF16 decode at 4K context: 32 q / 8 kv heads, head_dim 128, block 16",
    "b1_1k": "B=1 BF16 decode at 1K context: 32 q / 8 kv heads, head_dim 128, block 16",
    "b1_128": "B=1 BF16 decode at 128 keys: 32 q / 8 kv heads, head_dim 128, block 16",
    "fp8": "FP8-E4M3 KV decode: B=64, 16 q / 8 kv heads, head_dim 256, block 16, "
           "seq_lens U[1K, 8K], sliding window 4096",
    "nvfp4": "NVFP4 KV decode: B=16, 16 q / 2 kv heads, head_dim 512, block 16, "
             "seq_lens U[2K, 16K]",
}


def kv_bytes_per_token(w) -> int:
    """Algorithmic K+V bytes one attended token costs (all kv heads)."""
    D, Hkv = w.head_dim, w.num_kv_heads
    if w.kv_dtype == "bf16":
        return 2 * Hkv * D * 2
    if w.kv_dtype == "fp8":
        return 2 * Hkv * D
    return 2 * Hkv * (D // 2 + D // 16)


def attended_tokens(w) -> int:
    L = w.seq_lens.astype(np.int64)
    if w.sliding_window > 0:
        return int(np.minimum(L, w.sliding_window).sum())
    return int(L.sum())


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_splitk_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


class Layers:
    """NL layers' K/V pools of one workload, written by the library's cache write."""

    def __init__(self, w, num_layers=None, dev="cuda:0"):
        import torch
        import paged_kv_decode_splitk_amd as pkd
        self.w, self.dev = w, torch.device(dev)
        B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
        fmt = w.kv_dtype
        if fmt == "bf16":
            self.page_units = bs * Hkv * D
            pool_dtype = torch.int16
            page_bytes = self.page_units * 2
        elif fmt == "fp8":
            self.page_units = bs * Hkv * D
            pool_dtype = torch.uint8
            page_bytes = self.page_units
        else:
            self.block_stride, self.data_section = pkd.nvfp4_default_sections(Hkv, D, bs)
            self.page_units = self.block_stride
            pool_dtype = torch.uint8
            page_bytes = self.page_units
        pool_bytes = 2 * w.num_pages * page_bytes
        if num_layers is None:
            num_layers = max(2, int(np.ceil(4 * MALL_BYTES / pool_bytes)))
        self.num_layers = num_layers
        self.pool_bytes = pool_bytes

        def u16(a):
            return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(self.dev)

        key = u16(w.k_bits.reshape(w.num_tokens, -1))
        val = u16(w.v_bits.reshape(w.num_tokens, -1))
        slots = torch.from_numpy(w.slot_mapping).to(self.dev)
        self.k_scale = self.v_scale = 1.0
        if fmt == "fp8":          # calibration: absmax of K, then V, scale = absmax / 448
            amax = torch.zeros(2, dtype=torch.float32, device=self.dev)
            pkd.bf16_absmax(key, amax[0:1])
            pkd.bf16_absmax(val, amax[1:2])
            a = amax.cpu().numpy()
            self.k_scale = float(np.float32(a[0]) / np.float32(448.0))
            self.v_scale = float(np.float32(a[1]) / np.float32(448.0))
        self.k, self.v = [], []
        for _ in range(num_layers):
            kp = torch.zeros(w.num_pages * self.page_units, dtype=pool_dtype, device=self.dev)
            vp = torch.zeros_like(kp)
            self._write(key, val, kp, vp, slots)
            self.k.append(kp)
            self.v.append(vp)
        last = w.last_token_index()
        assert (last >= 0).all(), "every sequence of a decode step appends one token"
        self.new_key = key[torch.from_numpy(last).to(self.dev)].contiguous()
        self.new_val = val[torch.from_numpy(last).to(self.dev)].contiguous()
        self.new_slots = slots[torch.from_numpy(last).to(self.dev)].contiguous()
        del key, val, slots
        self.q = u16(w.q_bits.reshape(-1))
        self.bt = torch.from_numpy(w.block_tables).to(self.dev)
        self.lens = torch.from_numpy(w.seq_lens).to(self.dev)
        cus = torch.cuda.get_device_properties(self.dev).multi_processor_count
        self.num_splits = pkd.paged_decode_num_splits(B, Hq, Hkv, w.max_blocks_per_seq, bs,
                                                      w.sliding_window, cus)
        self.ws = torch.empty(pkd.paged_decode_workspace_bytes(B, Hq, D, self.num_splits) // 4,
                              dtype=torch.float32, device=self.dev)
        self.out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=self.dev)
        torch.cuda.synchronize()

    def _write(self, key, val, kp, vp, slots):
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        args = (key, val, kp, vp, slots, w.num_kv_heads, w.head_dim, w.block_size)
        if w.kv_dtype == "bf16":
            pkd.reshape_and_cache_bf16(*args)
        elif w.kv_dtype == "fp8":
            pkd.reshape_and_cache_fp8(*args, self.k_scale, self.v_scale)
        else:
            pkd.reshape_and_cache_nvfp4(*args, self.block_stride, self.data_section)

    def splitk(self, layer):
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        common = (self.q, self.k[layer], self.v[layer], self.ws, self.bt, self.lens,
                  w.max_blocks_per_seq, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                  float(w.scale), self.num_splits)
        qs = w.num_q_heads * w.head_dim
        if w.kv_dtype == "bf16":
            pkd.paged_decode_attn_splitk_bf16(*common, qs, w.num_seqs, w.sliding_window)
        elif w.kv_dtype == "fp8":
            pkd.paged_decode_attn_splitk_fp8(*common, self.k_scale, self.v_scale, qs,
                                             self.page_units, w.num_seqs, w.sliding_window)
        else:
            pkd.paged_decode_attn_splitk_nvfp4(*common, qs, self.block_stride, self.data_section,
                                               w.num_seqs, w.sliding_window)

    def decode(self, layer):
        """The whole-decode call with num_splits 1: one wave per row writes the output."""
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        common = (self.q, self.k[layer], self.v[layer], self.out, self.bt, self.lens,
                  w.max_blocks_per_seq, w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                  w.block_size, float(w.scale))
        tail = dict(sliding_window=w.sliding_window, workspace=None, num_splits=1)
        qs = w.num_q_heads * w.head_dim
        if w.kv_dtype == "bf16":
            pkd.paged_decode_attn_bf16(*common, qs, **tail)
        elif w.kv_dtype == "fp8":
            pkd.paged_decode_attn_fp8(*common, self.k_scale, self.v_scale, qs, self.page_units,
                                      **tail)
        else:
            pkd.paged_decode_attn_nvfp4(*common, qs, self.block_stride, self.data_section, **tail)

    def splitk_append(self, layer):
        """The split-K pass that first appends each sequence's new token."""
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        common = (self.q, self.new_key, self.new_val, self.k[layer], self.v[layer], self.ws,
                  self.bt, self.lens, w.max_blocks_per_seq, w.num_q_heads, w.num_kv_heads,
                  w.head_dim, w.block_size, float(w.scale), self.num_splits)
        qs = w.num_q_heads * w.head_dim
        if w.kv_dtype == "bf16":
            pkd.paged_decode_attn_splitk_append_bf16(*common, qs, w.num_seqs, w.sliding_window)
        elif w.kv_dtype == "fp8":
            pkd.paged_decode_attn_splitk_append_fp8(*common, self.k_scale, self.v_scale, qs,
                                                    self.page_units, w.num_seqs,
                                                    w.sliding_window)
        else:
            pkd.paged_decode_attn_splitk_append_nvfp4(*common, qs, self.block_stride,
                                                      self.data_section, w.num_seqs,
                                                      w.sliding_window)

    def step(self, layer):
        """The decode step in two launches: the split-K pass that appends the
        new token's K/V, then the combine pass."""
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        self.splitk_append(layer)
        pkd.paged_decode_attn_reduce(self.ws, self.out, self.lens, w.num_q_heads, w.head_dim,
                                     self.num_splits, w.num_seqs)

    def step_separate(self, layer):
        """The decode step in three launches: cache write, split-K, combine."""
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        self._write(self.new_key, self.new_val, self.k[layer], self.v[layer], self.new_slots)
        self.splitk(layer)
        pkd.paged_decode_attn_reduce(self.ws, self.out, self.lens, w.num_q_heads, w.head_dim,
                                     self.num_splits, w.num_seqs)

    def whole(self, layer, num_splits):
        """The whole-decode call without the cache write: num_splits 1 is the
        one-launch form; with the split heuristic's count the library runs the
        split pass and the combine, or the one-launch form for short rows."""
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        assert w.kv_dtype == "bf16"
        pkd.paged_decode_attn_bf16(self.q, self.k[layer], self.v[layer], self.out, self.bt,
                                   self.lens, w.max_blocks_per_seq, w.num_seqs, w.num_q_heads,
                                   w.num_kv_heads, w.head_dim, w.block_size, float(w.scale),
                                   w.num_q_heads * w.head_dim, sliding_window=w.sliding_window,
                                   workspace=self.ws if num_splits > 1 else None,
                                   num_splits=num_splits)

    def step_single(self, layer):
        """Write the new token's K/V, then the non-split decode (one launch)."""
        self._write(self.new_key, self.new_val, self.k[layer], self.v[layer], self.new_slots)
        self.decode(layer)


def _graph_time(fn, calls, reps):
    """ms per call of `fn(i)` for i in range(calls), captured in one HIP graph
    and replayed `reps` times between two events on the capturing stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    # one more untimed replay, then the timed ones queue behind it: the GPU
    # never waits for the host's graph launch inside the timed window
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / (reps * calls)


STEPS_PER_GRAPH = 32


def _steps_spread(fn, NL, steps):
    """p10 / p50 / p90 of the per-step time over graph replays: the same
    graphs of whole layer cycles as _steps_time, replayed `steps` steps' worth
    once more with an event pair around each replay (a pass of its own, so the
    timed run above carries no extra events)."""
    import torch
    per_graph = NL * max(1, -(-STEPS_PER_GRAPH // NL))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i % NL)
    g.replay()
    torch.cuda.synchronize()
    reps = max(8, steps // per_graph)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    g.replay()                                   # untimed; the timed replays queue behind it
    ev[0].record()
    for r in range(reps):
        g.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([ev[r].elapsed_time(ev[r + 1]) / per_graph for r in range(reps)])
    del g
    return {f"p{q}": float(np.percentile(per_step, q)) * 1e3 for q in (10, 50, 90)}


def _steps_time(fn, NL, steps):
    """ms per step of exactly `steps` steps fn(layer), cycling over the NL
    layers. The steps are captured as a model's layers are, many to a graph
    (whole cycles of at least STEPS_PER_GRAPH steps, plus one graph for the
    remainder), so that the host's graph launches stay off the step time;
    every kernel boundary inside a graph is still in it. The K steps run
    once untimed before the timed run."""
    import torch
    per_graph = NL * max(1, -(-STEPS_PER_GRAPH // NL))
    full, rem = divmod(steps, per_graph)
    graphs = []
    for count, n in ((full, per_graph), (1 if rem else 0, rem)):
        if count == 0:
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i % NL)
        g.replay()
        graphs.append((g, count))
    # the same K steps once untimed first: the GPU reaches the clocks it holds
    # under a steady decode load (the first graph replays after the host-side
    # capture run measurably slower). No host synchronization between them
    # and the timed run: its first graph is already queued when the untimed
    # steps end, as in a serving loop, so the host's launch latency stays
    # outside the timed window.
    torch.cuda.synchronize()
    for g, count in graphs:
        for _ in range(count):
            g.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for g, count in graphs:
        for _ in range(count):
            g.replay()
    b.record()
    torch.cuda.synchronize()
    del graphs
    return a.elapsed_time(b) / steps


def time_workload(name, steps, warmup, kernel_reps=100, single=True, whole=False):
    import torch
    import workloads
    w = workloads.make_workload(name)
    lay = Layers(w)
    NL = lay.num_layers
    # warm up eagerly (also loads the code objects), then graphs of one step per layer
    for i in range(max(1, warmup)):
        lay.step(i % NL)
        lay.step_separate(i % NL)
        if single:
            lay.step_single(i % NL)
    torch.cuda.synchronize()
    steps_run = steps
    t0 = time.perf_counter()
    ms_step = _steps_time(lay.step, NL, steps)
    wall = time.perf_counter() - t0
    spread = _steps_spread(lay.step, NL, steps)
    ms_sep = _steps_time(lay.step_separate, NL, steps)
    nan = float("nan")
    ms_single = _steps_time(lay.step_single, NL, steps) if single else nan
    # the kernels alone: back-to-back launches rotating over the layers
    single_ms = _graph_time(lambda i: lay.decode(i % NL), kernel_reps, 3) if single else nan
    k_ms = _graph_time(lambda i: lay.splitk_append(i % NL), kernel_reps, 3)
    plain_ms = _graph_time(lambda i: lay.splitk(i % NL), kernel_reps, 3)
    whole_one_ms = whole_ms = nan
    if whole:
        # the whole-decode call (no cache write), back to back over the layers
        for i in range(NL):
            lay.whole(i, 1)
            lay.whole(i, lay.num_splits)
        whole_one_ms = _graph_time(lambda i: lay.whole(i % NL, 1), kernel_reps, 3)
        whole_ms = _graph_time(lambda i: lay.whole(i % NL, lay.num_splits), kernel_reps, 3)

    kv_bytes = attended_tokens(w) * kv_bytes_per_token(w)
    gbs = lambda ms: kv_bytes / (ms * 1e-3) / 1e9
    res = dict(
        workload=name, description=DESCRIPTIONS.get(name, name), kv_dtype=w.kv_dtype,
        num_seqs=w.num_seqs, num_splits=lay.num_splits, layers_rotated=NL,
        kv_pool_bytes_per_layer=lay.pool_bytes, attended_tokens=attended_tokens(w),
        kv_bytes_per_step=kv_bytes, steps=steps_run, ms_per_step=ms_step,
        us_per_step=ms_step * 1e3, kv_gbs=gbs(ms_step), wall_s=wall,
        us_per_step_spread=spread,
        separate_write_us_per_step=ms_sep * 1e3, separate_write_kv_gbs=gbs(ms_sep),
        splitk_plain_us=plain_ms * 1e3, splitk_plain_gbs=gbs(plain_ms),
        non_split_us_per_step=ms_single * 1e3, non_split_kv_gbs=gbs(ms_single),
        non_split_kernel_us=single_ms * 1e3, non_split_kernel_gbs=gbs(single_ms),
        splitk_us=k_ms * 1e3, splitk_gbs=gbs(k_ms),
        whole_decode_us=whole_ms * 1e3, whole_decode_one_launch_us=whole_one_ms * 1e3,
        k_scale=lay.k_scale, v_scale=lay.v_scale,
    )
    res["pct_of_peak"] = 100.0 * res["kv_gbs"] / PEAK_HBM_GBS
    del lay
    torch.cuda.empty_cache()
    return res, w


def verify_tokens(w, q_len) -> int:
    """Keys the rows of a causal q_len-token block read: the whole sequence,
    or with a window W the last W + q_len - 1 keys."""
    L = w.seq_lens.astype(np.int64)
    if w.sliding_window > 0:
        return int(np.minimum(L, w.sliding_window + q_len - 1).sum())
    return int(L.sum())


class VerifyBlock:
    """A causal q_len-token query block per sequence over a workload's
    layers (speculative verify / chunked prefill): the multi-token call at
    the split count the library's heuristic picks."""

    def __init__(self, lay, q_len):
        import torch
        import paged_kv_decode_splitk_amd as pkd
        import workloads
        w = self.w = lay.w
        self.lay, self.q_len = lay, q_len
        B, Hq, D = w.num_seqs, w.num_q_heads, w.head_dim
        qb = workloads.query_block(w, q_len, seed=1)
        self.q = torch.from_numpy(qb.reshape(-1).view(np.int16)).to(lay.dev)
        cus = torch.cuda.get_device_properties(lay.dev).multi_processor_count
        self.num_splits = pkd.paged_prefill_num_splits(B, q_len, Hq, w.num_kv_heads,
                                                       w.max_blocks_per_seq, w.block_size, True,
                                                       w.sliding_window, cus)
        self.ws = torch.empty(pkd.paged_decode_workspace_bytes(B, Hq * q_len, D,
                                                               self.num_splits) // 4,
                              dtype=torch.float32, device=lay.dev)
        self.out = torch.empty((B, q_len, Hq, D), dtype=torch.bfloat16, device=lay.dev)

    def call(self, layer):
        import paged_kv_decode_splitk_amd as pkd
        w, lay = self.w, self.lay
        common = (self.q, lay.k[layer], lay.v[layer], self.out, lay.bt, lay.lens,
                  w.max_blocks_per_seq, w.num_seqs, self.q_len, w.num_q_heads, w.num_kv_heads,
                  w.head_dim, w.block_size, float(w.scale))
        tail = dict(causal=True, sliding_window=w.sliding_window, workspace=self.ws,
                    num_splits=self.num_splits)
        if w.kv_dtype == "bf16":
            pkd.paged_prefill_attn_bf16(*common, **tail)
        elif w.kv_dtype == "fp8":
            pkd.paged_prefill_attn_fp8(*common, lay.k_scale, lay.v_scale, lay.page_units, **tail)
        else:
            pkd.paged_prefill_attn_nvfp4(*common, lay.block_stride, lay.data_section, **tail)

    def reduce(self, layer):
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        pkd.paged_decode_attn_reduce(self.ws, self.out, self.lay.lens,
                                     w.num_q_heads * self.q_len, w.head_dim, self.num_splits,
                                     w.num_seqs)


def time_verify(name, q_lens, steps, warmup, kernel_reps=100):
    """us per multi-token call (split-K pass + combine, HIP-graph replay over
    the layers) for each q_len, and the split-K pass alone (the call minus
    the combine, both timed back to back)."""
    import torch
    import workloads
    w = workloads.make_workload(name)
    lay = Layers(w)
    NL = lay.num_layers
    res = {}
    for n in q_lens:
        vb = VerifyBlock(lay, n)
        for i in range(max(1, warmup)):
            vb.call(i % NL)
        torch.cuda.synchronize()
        ms = _steps_time(vb.call, NL, steps)
        red_ms = _graph_time(lambda i: vb.reduce(i % NL), kernel_reps, 3)
        kv_bytes = verify_tokens(w, n) * kv_bytes_per_token(w)
        split_us = (ms - red_ms) * 1e3
        chunks = -(-(w.group * n) // 16)
        res[f"{name}_q{n}"] = dict(
            q_len=n, causal=True, num_splits=vb.num_splits, query_rows=w.num_seqs * n * w.num_q_heads,
            column_chunks_per_kv_head=chunks, kv_bytes_per_step=kv_bytes,
            us_per_step=ms * 1e3, kv_gbs=kv_bytes / (ms * 1e-3) / 1e9,
            pct_of_peak=100.0 * kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            combine_us=red_ms * 1e3, splitk_us=split_us,
            splitk_gbs=kv_bytes / (split_us * 1e-6) / 1e9,
            query_tokens_per_s=w.num_seqs * n / (ms * 1e-3))
        del vb
    del lay
    torch.cuda.empty_cache()
    return res


class ContigLayers:
    """A workload's K/V as contiguous (b, h, l, d) or (b, l, h, d) tensors
    with l = the block-table capacity, NL layers of them (rotated like the
    paged pools), and the contiguous-K/V call over them (decode, q_len 1)."""

    def __init__(self, w, layout="bhld", dev="cuda:0"):
        import torch
        import paged_kv_decode_splitk_amd as pkd
        assert w.kv_dtype == "bf16", "contiguous timing: BF16 workloads"
        self.w, self.dev, self.layout = w, torch.device(dev), layout
        B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
        self.Lmax = w.max_blocks_per_seq * w.block_size
        per_layer = 2 * B * self.Lmax * Hkv * D * 2
        self.num_layers = max(2, int(np.ceil(4 * MALL_BYTES / per_layer)))
        self.pool_bytes = per_layer
        rows = torch.from_numpy(w.token_seq.astype(np.int64) * self.Lmax +
                                w.token_pos.astype(np.int64)).to(self.dev)

        def dense(bits):
            src = torch.from_numpy(bits.reshape(w.num_tokens, -1).view(np.int16)).to(self.dev)
            t = torch.zeros((B * self.Lmax, Hkv * D), dtype=torch.int16, device=self.dev)
            t[rows] = src
            t = t.view(B, self.Lmax, Hkv, D)
            if layout == "bhld":
                t = t.permute(0, 2, 1, 3).contiguous()
            return t.reshape(-1)

        self.k = [dense(w.k_bits) for _ in range(self.num_layers)]
        self.v = [dense(w.v_bits) for _ in range(self.num_layers)]
        self.kv_strides = pkd.layout_strides(layout, B, self.Lmax, Hkv, D)
        self.q = torch.from_numpy(w.q_bits.reshape(-1).view(np.int16)).to(self.dev)
        self.lens = torch.from_numpy(w.seq_lens).to(self.dev)
        cus = torch.cuda.get_device_properties(self.dev).multi_processor_count
        self.num_splits = pkd.paged_decode_num_splits(B, Hq, Hkv, w.max_blocks_per_seq,
                                                      w.block_size, w.sliding_window, cus)
        self.ws = torch.empty(pkd.paged_decode_workspace_bytes(B, Hq, D, self.num_splits) // 4,
                              dtype=torch.float32, device=self.dev)
        self.out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=self.dev)
        torch.cuda.synchronize()

    def call(self, layer):
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
        qs = (Hq * D, Hq * D, D)
        pkd.contig_kv_attn_bf16(self.q, self.k[layer], self.v[layer], self.out, self.lens, B, 1,
                                self.Lmax, Hq, Hkv, D, float(w.scale), qs, self.kv_strides,
                                self.kv_strides, qs, causal=True,
                                sliding_window=w.sliding_window, workspace=self.ws,
                                num_splits=self.num_splits)

    def reduce(self, layer):
        import paged_kv_decode_splitk_amd as pkd
        w = self.w
        pkd.paged_decode_attn_reduce(self.ws, self.out, self.lens, w.num_q_heads, w.head_dim,
                                     self.num_splits, w.num_seqs)


def time_contig(name, layout, steps, warmup, kernel_reps=100):
    """us per contiguous-K/V decode call (split-K pass + combine, graph
    replay over the layers) and the split-K pass alone (call minus combine)."""
    import torch
    import workloads
    w = workloads.make_workload(name)
    cl = ContigLayers(w, layout)
    NL = cl.num_layers
    for i in range(max(1, warmup)):
        cl.call(i % NL)
    torch.cuda.synchronize()
    ms = _steps_time(cl.call, NL, steps)
    red_ms = _graph_time(lambda i: cl.reduce(i % NL), kernel_reps, 3)
    kv_bytes = attended_tokens(w) * kv_bytes_per_token(w)
    split_us = (ms - red_ms) * 1e3
    res = dict(layout=layout, num_splits=cl.num_splits, layers_rotated=NL,
               kv_bytes_per_step=kv_bytes, us_per_step=ms * 1e3,
               kv_gbs=kv_bytes / (ms * 1e-3) / 1e9,
               pct_of_peak=100.0 * kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
               combine_us=red_ms * 1e3, splitk_us=split_us,
               splitk_gbs=kv_bytes / (split_us * 1e-6) / 1e9)
    del cl
    torch.cuda.empty_cache()
    return res


def time_aux(reps=10):
    """The two steps off the decode loop's timed path, each against HBM:
    bf16_absmax over the FP8 workload's whole K tensor (the calibration read),
    and reshape_and_cache_{bf16,fp8,nvfp4} writing every token of the llama8b
    batch into a fresh pool through its slot mapping. Seeded synthetic BF16
    values on the device; `reps` back-to-back launches between two events."""
    import torch
    import paged_kv_decode_splitk_amd as pkd
    import workloads
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    res = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3          # us per launch

    wf = workloads.make_workload("fp8", with_kv=False)
    n = int(wf.seq_lens.astype(np.int64).sum()) * wf.num_kv_heads * wf.head_dim
    x = torch.randn(n, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    us = timed(lambda: pkd.bf16_absmax(x.view(torch.int16), amax))
    res["bf16_absmax"] = dict(elements=n, us=us, gbs=2 * n / (us * 1e-6) / 1e9,
                              pct_of_peak=100.0 * 2 * n / (us * 1e-6) / 1e9 / PEAK_HBM_GBS)
    del x

    w = workloads.make_workload("llama8b", with_kv=False)
    T, Hkv, D, bs = w.num_tokens, w.num_kv_heads, w.head_dim, w.block_size
    key = torch.randn((T, Hkv * D), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    val = torch.randn((T, Hkv * D), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    slots = torch.from_numpy(w.slot_mapping).to(dev)
    args = (key, val)
    for fmt in ("bf16", "fp8", "nvfp4"):
        if fmt == "bf16":
            page, dt, out_b = bs * Hkv * D, torch.int16, 2.0
        elif fmt == "fp8":
            page, dt, out_b = bs * Hkv * D, torch.uint8, 1.0
        else:
            stride, data = pkd.nvfp4_default_sections(Hkv, D, bs)
            page, dt, out_b = stride, torch.uint8, 0.5 + 1.0 / 16
        kp = torch.zeros(w.num_pages * page, dtype=dt, device=dev)
        vp = torch.zeros_like(kp)
        tail = (slots, Hkv, D, bs)
        if fmt == "bf16":
            fn = lambda: pkd.reshape_and_cache_bf16(*args, kp, vp, *tail)
        elif fmt == "fp8":
            fn = lambda: pkd.reshape_and_cache_fp8(*args, kp, vp, *tail, 0.01, 0.01)
        else:
            fn = lambda: pkd.reshape_and_cache_nvfp4(*args, kp, vp, *tail, stride, data)
        us = timed(fn)
        nbytes = 2 * T * Hkv * D * (2 + out_b)         # K and V: BF16 in, encoded out
        res[f"reshape_and_cache_{fmt}"] = dict(tokens=T, us=us, gbs=nbytes / (us * 1e-6) / 1e9,
                                               pct_of_peak=100.0 * nbytes / (us * 1e-6) / 1e9
                                               / PEAK_HBM_GBS)
        del kp, vp
    del key, val
    torch.cuda.empty_cache()
    return res


def counter_run(name, calls=20):
    """Only the split-K pass with the append, `calls` times over the layers
    (for rocprofv3 counter passes, which profile every dispatch)."""
    import torch
    import workloads
    w = workloads.make_workload(name)
    lay = Layers(w)
    torch.cuda.synchronize()
    for i in range(calls):
        lay.splitk_append(i % lay.num_layers)
    torch.cuda.synchronize()
    print(json.dumps({"counter_run": name, "calls": calls, "num_splits": lay.num_splits,
                      "kv_bytes_per_call": attended_tokens(w) * kv_bytes_per_token(w)}))


def trace_run(name, replays=6):
    """Only the graph-replayed decode step (split-K with append + combine),
    one graph of whole layer cycles replayed `replays` times after one
    untimed replay (for a rocprofv3 kernel trace: start, end and the gap
    between the two launches of each step)."""
    import torch
    import workloads
    w = workloads.make_workload(name)
    lay = Layers(w)
    NL = lay.num_layers
    per_graph = NL * max(1, -(-STEPS_PER_GRAPH // NL))
    for i in range(NL):
        lay.step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            lay.step(i % NL)
    g.replay()
    torch.cuda.synchronize()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    print(json.dumps({"trace_run": name, "steps_per_graph": per_graph, "replays": replays,
                      "num_splits": lay.num_splits}))


def traffic_record(name, tag):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary (profiles/traffic_<tag>_<workload>.txt), used
    only while the kernel sources still hash to what was profiled."""
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}_{name}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_hash") != source_hash():
        return None
    try:
        return float(rec["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def counters_record(name):
    """SQ-counter utilization of the split-K pass from the committed rocprofv3
    summary (profiles/counters_splitk_<workload>.txt), used only while the
    kernel sources still hash to what was profiled; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"counters_splitk_{name}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip().split()[0]
    if rec.get("source_hash") != source_hash():
        return None
    keys = ("valu_busy_pct_of_simd_cycles", "mfma_busy_pct_of_simd_cycles",
            "valu_insts_per_wave_tile", "wave_cycles_issuing_pct", "wave_cycles_waiting_any_pct",
            "lds_bank_conflict_cycles_pct_of_cu_cycles")
    try:
        out = {k: float(rec[k]) for k in keys}
    except (KeyError, ValueError):
        return None
    out["source"] = f"profiles/counters_splitk_{name}.txt"
    return out


def cpu_baseline(w, budget_s=12.0, max_seqs=None, k_scale=1.0, v_scale=1.0, max_reps=50):
    """The float64 oracle on the host: decode steps of a sample of the
    workload's sequences (the first `max_seqs`, or all), repeated until the
    time budget is spent, each sequence's page gather, dequantization and
    softmax attention timed; the sample's caches are written once before
    timing (in token chunks, untimed). Scaled to GB/s of attended KV."""
    import oracle
    from threadpoolctl import threadpool_info
    geom = oracle.CacheGeometry(w.kv_dtype, w.num_pages, w.block_size, w.num_kv_heads,
                                w.head_dim)
    kc, vc = oracle.new_cache(geom, 0), oracle.new_cache(geom, 0)
    nseq = w.num_seqs if max_seqs is None else min(int(max_seqs), w.num_seqs)
    seqs = list(range(nseq))
    tok = np.nonzero(np.isin(w.token_seq, seqs))[0]
    for i in range(0, tok.size, 4096):
        part = tok[i:i + 4096]
        oracle.reshape_and_cache(geom, w.k_bits[part], w.v_bits[part], kc, vc,
                                 w.slot_mapping[part], k_scale=k_scale, v_scale=v_scale)
    kv_bytes = attended_tokens(w) * kv_bytes_per_token(w)
    total_t, total_bytes, reps = 0.0, 0, 0
    lens = w.seq_lens.astype(np.int64)
    while total_t < budget_s and reps < max_reps:
        for b in seqs:
            t0 = time.perf_counter()
            oracle.paged_decode_attention(geom, w.q_bits, kc, vc, w.block_tables, w.seq_lens,
                                          w.num_q_heads, w.scale, sliding_window=w.sliding_window,
                                          k_scale=k_scale, v_scale=v_scale, seqs=[b])
            dt = time.perf_counter() - t0
            total_t += dt
            L = lens[b] if w.sliding_window <= 0 else min(lens[b], w.sliding_window)
            total_bytes += int(L) * kv_bytes_per_token(w)
            if total_t >= budget_s:
                break
        reps += 1
    blas = [p.get("num_threads", 1) for p in threadpool_info()]
    threads = max(blas) if blas else 1
    sample = (f"{w.name}: float64 NumPy oracle decode (page gather, dequant, softmax attention) "
              f"of {'all ' + str(nseq) if nseq == w.num_seqs else 'the first ' + str(nseq) + ' of ' + str(w.num_seqs)} "
              f"sequences, {total_bytes / kv_bytes:.2f} steps' worth of KV in {total_t:.1f} s; "
              f"cache write untimed; {len(os.sched_getaffinity(0))} host cores visible, BLAS "
              f"threads {threads}")
    return dict(value=total_bytes / total_t / 1e9, unit="GB/s", cores=int(threads),
                kind="oracle", sample=sample, s_per_step=total_t * kv_bytes / total_bytes)


# Bounded oracle samples beside each extra workload: (seconds, sequences).
CPU_SAMPLES = {"b1_32k": (6.0, None), "fp8": (6.0, 8), "nvfp4": (6.0, 4),
               "b1_128": (0.5, None), "b1_1k": (1.5, None), "b1_4k": (1.5, None), "b1_8k": (1.5, None),
               "b1_16k": (2.0, None)}


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the rocprof byte counters."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--extra", nargs="*", default=["b1_32k", "fp8", "nvfp4"])
    ap.add_argument("--sweep", nargs="*", default=["b1_128", "b1_1k", "b1_4k", "b1_8k", "b1_16k"],
                    help="B=1 context sweep: step, split-K kernel and whole-decode call per "
                         "context")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-single", action="store_true",
                    help="skip the non-split decode timings (profiles then see only the "
                         "split-K launches of the kernel)")
    ap.add_argument("--verify", nargs="*", default=["llama8b:4", "llama8b:8"],
                    help="multi-token (causal query block) timings, as workload:q_len")
    ap.add_argument("--contig", nargs="*", default=["llama8b:bhld"],
                    help="contiguous-K/V decode timings, as workload:layout (BF16)")
    ap.add_argument("--verify-only", action="store_true",
                    help="only the --verify timings (for kernel statistics of that call)")
    ap.add_argument("--counter-run", action="store_true",
                    help="only run the split-K pass of --workload 20 times")
    ap.add_argument("--trace-run", action="store_true",
                    help="only replay graphs of the decode step of --workload (kernel trace)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the paged decode path runs on a single MI355X "
              "and has no multi-GPU mode; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    if args.counter_run:
        counter_run(args.workload)
        return
    if args.trace_run:
        trace_run(args.workload)
        return
    if args.verify_only:
        out = {}
        for spec in args.verify:
            nm, n = spec.split(":")
            out.update(time_verify(nm, [int(n)], args.steps, args.warmup))
        for spec in args.contig:
            nm, lay = spec.split(":")
            out[f"contig_{nm}_{lay}"] = time_contig(nm, lay, args.steps, args.warmup)
        print(json.dumps({"verify": out}))
        return
    print(f"bench: {args.workload} steps={args.steps} warmup={args.warmup}", file=sys.stderr,
          flush=True)
    main_res, w = time_workload(args.workload, args.steps, args.warmup, single=not args.no_single)
    print(f"bench: {args.workload} {main_res['us_per_step']:.2f} us/step "
          f"{main_res['kv_gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    extras = {}
    def side_baseline(name, r, wl):
        if args.no_cpu_baseline:
            return None
        budget, nseq = CPU_SAMPLES.get(name, (6.0, 8))
        cb = cpu_baseline(wl, budget_s=budget, max_seqs=nseq, k_scale=r["k_scale"],
                          v_scale=r["v_scale"])
        print(f"bench: {name} oracle {cb['value']:.3f} GB/s ({cb['s_per_step']:.3f} s/step)",
              file=sys.stderr, flush=True)
        return cb

    for name in args.extra:
        r, wx = time_workload(name, args.steps, args.warmup, single=not args.no_single)
        extras[name] = {k: r[k] for k in ("us_per_step", "us_per_step_spread", "kv_gbs",
                                          "pct_of_peak",
                                          "separate_write_us_per_step",
                                          "separate_write_kv_gbs",
                                          "splitk_plain_us", "splitk_plain_gbs",
                                          "non_split_us_per_step",
                                          "non_split_kv_gbs",
                                          "non_split_kernel_us", "non_split_kernel_gbs",
                                          "splitk_us", "splitk_gbs", "num_splits",
                                          "kv_bytes_per_step", "layers_rotated", "kv_dtype")}
        print(f"bench: {name} {r['us_per_step']:.2f} us/step {r['kv_gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)
        extras[name]["cpu_baseline"] = side_baseline(name, r, wx)
        del wx

    sweep = {}
    for name in args.sweep:
        r, wx = time_workload(name, args.steps, args.warmup, single=False, whole=True)
        sweep[name] = {k: r[k] for k in ("us_per_step", "kv_gbs", "pct_of_peak", "splitk_us",
                                         "splitk_gbs", "splitk_plain_us", "splitk_plain_gbs",
                                         "whole_decode_us", "whole_decode_one_launch_us",
                                         "num_splits", "kv_bytes_per_step")}
        print(f"bench: sweep {name} {r['us_per_step']:.2f} us/step, split-K "
              f"{r['splitk_plain_us']:.2f} us {r['splitk_plain_gbs']:.0f} GB/s, whole decode "
              f"{r['whole_decode_us']:.2f} us (one launch {r['whole_decode_one_launch_us']:.2f})",
              file=sys.stderr, flush=True)
        sweep[name]["cpu_baseline"] = side_baseline(name, r, wx)
        del wx
    verify = {}
    by_name = {}
    for spec in args.verify:
        nm, n = spec.split(":")
        by_name.setdefault(nm, []).append(int(n))
    for nm, ns in by_name.items():
        r = time_verify(nm, ns, args.steps, args.warmup)
        for k, v in r.items():
            print(f"bench: verify {k} {v['us_per_step']:.2f} us/step {v['kv_gbs']:.0f} GB/s",
                  file=sys.stderr, flush=True)
        verify.update(r)
    contig = {}
    for spec in args.contig:
        nm, lay = spec.split(":")
        r = time_contig(nm, lay, args.steps, args.warmup)
        print(f"bench: contiguous {nm} {lay} {r['us_per_step']:.2f} us/step "
              f"{r['kv_gbs']:.0f} GB/s", file=sys.stderr, flush=True)
        contig[f"{nm}_{lay}"] = r

    aux = time_aux()
    print("bench: aux " + ", ".join(f"{k} {v['us']:.1f} us {v['gbs']:.0f} GB/s"
                                    for k, v in aux.items()), file=sys.stderr, flush=True)

    # the step's dominant kernel: the split-K pass (with the append)
    fmt = main_res["kv_dtype"]
    kernel, us, tag = f"paged_decode_attn_splitk_append_{fmt}", main_res["splitk_us"], "splitk"
    achieved = main_res["kv_bytes_per_step"] / (us * 1e-6) / 1e9
    traffic = traffic_record(args.workload, tag)
    roofline = dict(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=achieved / PEAK_HBM_GBS, traffic=traffic, kernel=kernel,
                    algorithmic_bytes_per_launch=main_res["kv_bytes_per_step"],
                    avg_launch_us=us, sq_counters=counters_record(args.workload))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, budget_s=args.cpu_budget)
    line = {
        "metric": METRIC,
        "value": main_res["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": main_res["steps"],
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "us_per_step": main_res["us_per_step"],
        "pct_of_peak": main_res["pct_of_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res["kv_dtype"],
        "data": "synthetic (seeded N(0,1) q/k/v, shuffled page pool)",
        "config": {
            "workload": main_res["description"],
            "num_splits": main_res["num_splits"],
            "layers_rotated": main_res["layers_rotated"],
            "kv_bytes_per_step": main_res["kv_bytes_per_step"],
            "step": "split-KV pass that first appends the new token's K/V (the cache write) "
                    "+ combine pass, HIP-graph replay",
        },
        "us_per_step_spread": main_res["us_per_step_spread"],
        "separate_write_step": {k: main_res[k] for k in ("separate_write_us_per_step",
                                                          "separate_write_kv_gbs")},
        "non_split_step": {k: main_res[k] for k in ("non_split_us_per_step",
                                                     "non_split_kv_gbs")},
        "kernels": {k: main_res[k] for k in ("non_split_kernel_us", "non_split_kernel_gbs",
                                             "splitk_plain_us", "splitk_plain_gbs", "splitk_us",
                                             "splitk_gbs")},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    for name, r in extras.items():
        line[name] = r
        # the same roofline record for the extra workload's split-K pass (with the append)
        ach = r["kv_bytes_per_step"] / (r["splitk_us"] * 1e-6) / 1e9
        line[name]["roofline"] = dict(
            bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s", frac=ach / PEAK_HBM_GBS,
            traffic=traffic_record(name, "splitk"),
            kernel=f"paged_decode_attn_splitk_append_{r['kv_dtype']}",
            algorithmic_bytes_per_launch=r["kv_bytes_per_step"], avg_launch_us=r["splitk_us"],
            sq_counters=counters_record(name))
    if sweep:
        line["b1_sweep"] = sweep
    if verify:
        line["verify"] = verify
    if contig:
        line["contiguous_kv"] = contig
    line["aux_kernels"] = aux
    print(json.dumps(line))


if __name__ == "__main__":
    main()
