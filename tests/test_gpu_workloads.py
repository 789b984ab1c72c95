"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.

The GPU runs every linear at full size (the seven projections of a decoder
block in one grouped launch, the 151936 x 2560 head, the mixed-width
down_proj).  The oracle computes a sample of output rows (rows are
independent, so a sample is exact for those rows): codes, scales, zeros and
packed words of the sampled rows must match bit for bit, and the sampled
outputs must meet the tolerance.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_rht_amd as dq
import workloads as W
from oracle import linear as OL
from oracle import pack as OP
from oracle import rtn as OR

from gpu_util import check_close, dev, dev_u32, host_f16_bits, host_u32, say

pytestmark = pytest.mark.gpu

SEED = 0
SAMPLE = 48


def _sample_rows(n, rng):
    rows = set(rng.choice(n, min(n, SAMPLE), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(rows))


def _check_rows(qw, lin, w_rows, rows, x, signs, bits_rows, y_gpu, label):
    """Bit-exact codes/scales/zeros/words and toleranced outputs on sampled rows."""
    q, s, z = OR.prepare(w_rows, signs, bits_rows)
    # scales and zeros
    sg = host_f16_bits(qw.scales)[rows]
    zg = host_f16_bits(qw.zeros)[rows]
    assert np.array_equal(sg, s.view(np.uint16)), label
    assert np.array_equal(zg, z.view(np.uint16)), label
    # packed words of the sampled rows
    words = host_u32(qw.codes)
    if lin.bits:
        wpr = OP.words_per_row(lin.bits, lin.k)
        for i, r in enumerate(rows):
            assert np.array_equal(words[r * wpr:(r + 1) * wpr], OP.pack_row(q[i], lin.bits)), (label, r)
    else:
        off = qw.block_off.cpu().numpy()
        for i, r in enumerate(rows):
            b = int(bits_rows[i])
            wpr = OP.words_per_row(b, lin.k)
            st = int(off[r // 64]) + (r % 64) * wpr
            assert np.array_equal(words[st:st + wpr], OP.pack_row(q[i], b)), (label, r)
    ref = OL.linear(q, s, z, x, signs if lin.rht else None)
    return check_close(y_gpu[:, rows], ref, label)


def _block(name, m):
    wl = W.WORKLOADS[name]
    lins = [l for l in wl.linears if l.bits != 0 and not l.out_f32]
    qws, xs, hosts = [], [], []
    for i, lin in enumerate(lins):
        w, x, signs, _ = W.linear_inputs(SEED, wl.wid, i, lin, m)
        qws.append(dq.quantize_weight(dev(w), lin.bits, dev_u32(signs)))
        xs.append(dev(x))
        hosts.append((w, x, signs))
    ys = dq.wq_linear_batch(qws, xs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(123)
    for i, lin in enumerate(lins):
        w, x, signs = hosts[i]
        rows = _sample_rows(lin.n, rng)
        rel, mx = _check_rows(qws[i], lin, w[rows], rows, x, signs, np.full(len(rows), lin.bits),
                              ys[i].float().cpu().numpy(), f"{name} {lin.name} m={m}")
        say(f"  {lin.name}: rel-L2 {rel:.2e} max/rms {mx:.2e}")


def test_single_int4_full():
    say("single_int4 1024->512 m=1, full oracle")
    wl = W.WORKLOADS["single_int4"]
    lin = wl.linears[0]
    w, x, signs, _ = W.linear_inputs(SEED, wl.wid, 0, lin, 1)
    q, s, z = OR.prepare(w, signs, 4)
    qw = dq.quantize_weight(dev(w), 4, dev_u32(signs))
    torch.cuda.synchronize()
    assert np.array_equal(host_u32(qw.codes).reshape(lin.n, -1), OP.pack(q, 4))
    y = dq.wq_linear(qw, dev(x))
    check_close(y.float().cpu().numpy(), OL.linear(q, s, z, x, signs), "single_int4")


@pytest.mark.parametrize("m", [1, 4])
def test_block_int4(m):
    say(f"block_int4 m={m}")
    _block("block_int4", m)


@pytest.mark.parametrize("m", [1, 4, 16])
def test_block_int3(m):
    say(f"block_int3 m={m}")
    _block("block_int3", m)


def test_block_int6():
    say("block_int6 m=1")
    _block("block_int6_head_int8", 1)


@pytest.mark.parametrize("m", [1, 4])
def test_head_int8_fp32_logits(m):
    # m = 1 is the configured case; m = 4 runs the head on the batch tiles
    # (594 rows per workgroup, fp32 outputs)
    say(f"head int8 151936x2560 m={m} fp32 out, no rotation")
    wl = W.WORKLOADS["block_int6_head_int8"]
    idx = len(wl.linears) - 1
    lin = wl.linears[idx]
    w, x, _, _ = W.linear_inputs(SEED, wl.wid, idx, lin, m)
    qw = dq.quantize_weight(dev(w), 8, None)
    y = dq.wq_linear(qw, dev(x), torch.float32, fuse_rht=False)
    torch.cuda.synchronize()
    rows = _sample_rows(lin.n, np.random.default_rng(9))
    rel, mx = _check_rows(qw, lin, w[rows], rows, x, None, np.full(len(rows), 8), y.cpu().numpy(), "head")
    say(f"  head: rel-L2 {rel:.2e} max/rms {mx:.2e}")
    del w


def test_mixed_down_proj_full():
    say("mixed 6/8 down_proj 9728->2560 m=1, full oracle")
    wl = W.WORKLOADS["prefill_and_mixed"]
    idx = len(wl.linears) - 1
    lin = wl.linears[idx]
    w, x, signs, sel = W.linear_inputs(SEED, wl.wid, idx, lin, 1)
    qw = dq.quantize_weight(dev(w), 0, dev_u32(signs), dev(sel))
    y = dq.wq_linear(qw, dev(x))
    torch.cuda.synchronize()
    rows = np.arange(lin.n)
    rel, mx = _check_rows(qw, lin, w, rows, x, signs, np.repeat(sel, 64), y.float().cpu().numpy(), "mixed")
    say(f"  mixed: rel-L2 {rel:.2e} max/rms {mx:.2e}")


def test_prefill_int4_m512():
    say("prefill int4 m=512 (matrix-core path)")
    wl = W.WORKLOADS["prefill_and_mixed"]
    m = 512
    rng = np.random.default_rng(321)
    for i, lin in enumerate(wl.linears[:-1]):
        w, x, signs, _ = W.linear_inputs(SEED, wl.wid, i, lin, m)
        qw = dq.quantize_weight(dev(w), 4, dev_u32(signs))
        y = dq.wq_linear(qw, dev(x))
        torch.cuda.synchronize()
        rows = _sample_rows(lin.n, rng)
        mrows = np.sort(rng.choice(m, 24, replace=False))
        q, s, z = OR.prepare(w[rows], signs, 4)
        ref = OL.linear(q, s, z, x[mrows], signs)
        rel, mx = check_close(y.float().cpu().numpy()[np.ix_(mrows, rows)], ref, f"prefill {lin.name}")
        say(f"  {lin.name}: rel-L2 {rel:.2e} max/rms {mx:.2e}")
