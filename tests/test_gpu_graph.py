"""Grouped calls captured in a HIP graph and replayed, through the C ABI.

A caller that captures wq_linear_batch once replays the same launches with
whatever its input buffers hold at replay time.  Every path is captured:
the batch-1 ring (int4 and the 8-bit ring with staged scales), the batch
tiles (arrangement pre-pass, then the row-quad kernel), the matrix cores
at 24 and 96 rows (rotation pre-pass, GEMM, split-K partial sums) and the
mixed 6/8 layout at batch 1 (workgroups placed by the host and found on the
device).  Each graph is replayed three times, with new activations written
into the captured input buffers before each replay and unrelated eager GPU
work and synchronisations between the replays; every replay must equal an
eager call on the same inputs bit for bit (the kernels are deterministic),
and the last one must meet the oracle's tolerance.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_rht_amd as dq
import workloads as W
from oracle import linear as OL
from oracle import rtn as OR

from gpu_util import check_close, dev, dev_u32, say

pytestmark = pytest.mark.gpu

# (label, bits, [(n, k), ...], m); bits 0 = mixed 6/8 with seeded selectors
CASES = [
    ("ring int4", 4, [(512, 2560), (256, 9728)], 1),
    ("ring int8 staged", 8, [(384, 2560), (130, 1152)], 1),
    ("batch tile", 4, [(512, 2560), (256, 9728)], 4),
    ("matrix cores 24", 4, [(512, 2560), (256, 9728)], 24),
    ("matrix cores 96", 3, [(300, 2560), (256, 9728)], 96),
    ("mixed host placement", 0, [(640, 2560)], 1),
    ("mixed device search", 0, [(640, 2560)], 1),
]


def _weights(bits, shapes, seed, host_widths):
    qs, hosts = [], []
    for i, (n, k) in enumerate(shapes):
        rng = np.random.default_rng(seed + i)
        w = W.weight(k, n, rng)
        signs = W.sign_bits(k, rng)
        sel = W.block_selector(n, rng, 0.3) if bits == 0 else None
        bits_rows = np.repeat(sel, 64) if bits == 0 else bits
        q, s, z = OR.prepare(w, signs, bits_rows)
        sel_d = dev(sel) if sel is not None else None
        packed, off = dq.wq_pack(dev(q), bits, sel_d)
        qs.append(dq.QWeight(bits, n, k, packed, dev(s), dev(z), dev_u32(signs), sel_d, off,
                             host_widths=host_widths))
        hosts.append((q, s, z, signs))
    return qs, hosts


@pytest.mark.parametrize("label,bits,shapes,m", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(label, bits, shapes, m):
    say(f"graph: {label} m={m}")
    qs, hosts = _weights(bits, shapes, 1400 + m + bits, host_widths="device" not in label)
    rng = np.random.default_rng(1500 + m)
    xs = [torch.empty((m, k), dtype=torch.float16, device="cuda") for (_, k) in shapes]
    ys = [torch.empty((m, n), dtype=torch.float16, device="cuda") for (n, _) in shapes]
    ye = [torch.empty_like(y) for y in ys]
    ws = dq.new_workspace(dq.wq_linear_batch_workspace(qs, m))
    captured = dq.BatchCall(qs, xs, ys, True, ws)
    eager = dq.BatchCall(qs, xs, ye, True, ws)

    def fill():
        vals = [W.activations(m, k, rng) for (_, k) in shapes]
        for x, v in zip(xs, vals):
            x.copy_(dev(v))
        return vals

    s = torch.cuda.Stream()
    fill()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        captured(s.cuda_stream)   # once before capture, outside it
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        captured(s.cuda_stream)
    scratch = torch.randn((1024, 1024), device="cuda")
    for r in range(3):
        vals = fill()
        scratch = torch.tanh(scratch @ scratch.T * 1e-3)   # unrelated eager work
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        eager()
        torch.cuda.synchronize()
        for (n, k), y, e in zip(shapes, ys, ye):
            assert torch.equal(y, e), f"{label}: replay {r} differs from the eager call (n={n} k={k} m={m})"
        say(f"  replay {r}: equal to the eager call")
    for (n, k), y, (q, sc, z, signs), x in zip(shapes, ys, hosts, vals):
        ref = OL.linear(q, sc, z, x, signs)
        rel, mx = check_close(y.float().cpu().numpy(), ref, f"{label} n={n} k={k} m={m}")
        say(f"  n={n} k={k}: rel-L2 {rel:.2e} max/rms {mx:.2e}")
    del g
