"""Writes tests/golden/tiny_decode.txt: the tiny paged decode workload (two
sequences of 17 and 40 tokens, 4 q / 2 kv heads, head_dim 64, block 16,
eight shuffled pages) with the CPU oracle's float64 output. The standalone
C++ test of the library reads it.

Inputs come from the seeded workload generator; the expected output comes
from the oracle only.

  python tests/golden/make_tiny_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def main(path=os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_decode.txt")):
    w = workloads.make_workload("tiny")
    geom = oracle.CacheGeometry("bf16", w.num_pages, w.block_size, w.num_kv_heads, w.head_dim)
    kc, vc = oracle.new_cache(geom, 0x7FC0), oracle.new_cache(geom, 0x7FC0)
    oracle.reshape_and_cache(geom, w.k_bits, w.v_bits, kc, vc, w.slot_mapping)
    out = oracle.paged_decode_attention(geom, w.q_bits, kc, vc, w.block_tables, w.seq_lens,
                                        w.num_q_heads, w.scale)
    hexs = lambda a: " ".join(f"{int(x):04x}" for x in np.asarray(a).reshape(-1))
    ints = lambda a: " ".join(str(int(x)) for x in np.asarray(a).reshape(-1))
    with open(path, "w") as f:
        f.write("# tiny paged decode: inputs from the seeded workload generator, output from the\n")
        f.write("# float64 CPU oracle (tests/golden/make_tiny_golden.py); one field per line:\n")
        f.write("# name, then values (BF16 bit patterns in hex, integers, or doubles)\n")
        f.write(f"dims {w.num_seqs} {w.num_q_heads} {w.num_kv_heads} {w.head_dim} {w.block_size} "
                f"{w.max_blocks_per_seq} {w.num_pages} {w.num_tokens}\n")
        f.write(f"scale {float(w.scale)!r}\n")
        f.write(f"seq_lens {ints(w.seq_lens)}\n")
        f.write(f"block_tables {ints(w.block_tables)}\n")
        f.write(f"slot_mapping {ints(w.slot_mapping)}\n")
        f.write(f"q {hexs(w.q_bits)}\n")
        f.write(f"k {hexs(w.k_bits)}\n")
        f.write(f"v {hexs(w.v_bits)}\n")
        f.write("out " + " ".join(f"{x:.17g}" for x in out.reshape(-1)) + "\n")
    print(path)


if __name__ == "__main__":
    main()
