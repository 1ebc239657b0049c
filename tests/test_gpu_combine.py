"""The combine (paged_decode_attn_reduce) on workspaces written on the host.

Each slot of a seeded workspace holds a partial (o, m, l): some slots hold no
keys (l = 0), an end marker (l < 0) follows the last piece, and the slots
after it hold stale values (NaN outputs, huge m, positive l) that must not
reach the result. Some sequences are empty (length 0, zeros out) and some
rows hold no key at all. Checked against the oracle's combine of the slots
before the marker, atol = rtol = 1e-2. The cases span every head dim, few
rows (the launch then splits a row's columns over several workgroups) and
many, and slot counts that need more than one round of value loads or more
than one chunk of (m, l) reads."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_splitk_amd as pkd
from gpu_cases import assert_close, dev, i32_to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, D, S, stop (None: every slot holds a piece, no marker)
    (1, 32, 128, 513, 129),
    (1, 32, 128, 513, 300),       # past the first round of value loads
    (1, 8, 512, 2000, 1500),      # several chunks of (m, l) reads
    (1, 1, 512, 4096, 4000),      # the most slots a call may have
    (1, 4, 64, 64, 64),
    (2, 3, 256, 100, None),
    (3, 5, 128, 9, 4),            # few rows, few slots
    (1, 2, 64, 1, None),          # one slot
    (64, 16, 128, 40, 17),        # many rows: one wave per row
    (16, 16, 512, 129, 33),       # many rows, more than 64 slots
    (40, 8, 64, 300, 250),
    (5, 40, 256, 70, 65),
]


def _workspace(B, Hq, D, S, stop, rng):
    """float32 [B][Hq][S][D + 2] and, per row, the number of slots before the marker."""
    ws = np.empty((B, Hq, S, D + 2), np.float32)
    stops = np.empty((B, Hq), np.int64)
    for b in range(B):
        for h in range(Hq):
            n = S if stop is None else min(S, max(0, stop - int(rng.integers(0, 3))))
            stops[b, h] = n
            o = rng.standard_normal((S, D)).astype(np.float32)
            m = (rng.standard_normal(S) * 3).astype(np.float32)
            l = rng.uniform(0.5, 50.0, S).astype(np.float32)
            empty = rng.random(S) < 0.15                     # pieces without keys
            l[empty] = 0.0
            m[empty] = -3.0e38
            if n < S:                                        # end marker, then stale slots
                l[n] = -1.0
                o[n + 1:] = np.nan
                m[n + 1:] = 1.0e30
                l[n + 1:] = 7.0
            ws[b, h, :, :D], ws[b, h, :, D], ws[b, h, :, D + 1] = o, m, l
    if B > 1:
        ws[0, 0, :, D + 1] = np.where(ws[0, 0, :, D + 1] > 0, 0.0, ws[0, 0, :, D + 1])  # no key
    return ws, stops


@pytest.mark.parametrize("B,Hq,D,S,stop", CASES)
def test_combine_of_host_partials(B, Hq, D, S, stop):
    print(f"[combine] B={B} Hq={Hq} D={D} S={S} stop={stop}", flush=True)
    rng = np.random.default_rng([B, Hq, D, S])
    ws, stops = _workspace(B, Hq, D, S, stop, rng)
    lens = rng.integers(1, 5000, B).astype(np.int32)
    if B > 2:
        lens[1] = 0                                          # an empty sequence
    ref = np.zeros((B, Hq, D))
    for b in range(B):
        if lens[b] <= 0:
            continue
        for h in range(Hq):
            n = int(stops[b, h])
            if n:
                ref[b, h] = oracle.combine_partials(ws[b, h, :n, :D].astype(np.float64),
                                                    ws[b, h, :n, D].astype(np.float64),
                                                    ws[b, h, :n, D + 1].astype(np.float64))
    wt = torch.from_numpy(ws.reshape(-1)).to(dev())
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=dev())
    pkd.paged_decode_attn_reduce(wt, out, i32_to_dev(lens), Hq, D, S, B)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert_close(got, ref, f"combine B={B} Hq={Hq} D={D} S={S}")
