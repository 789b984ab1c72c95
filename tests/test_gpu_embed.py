"""GPU parity of the tied-embedding gather (wq_embed) against the oracle.

A gathered row is the dequantised table row rounded once, so the library
must match the oracle bit for bit in fp16 and in fp32: small tables of every
uniform width with ragged ids (duplicates, the first and last row, ids
outside the table), strided outputs, and the 151936 x 2560 int8 head table
on sampled rows.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_rht_amd as dq
import workloads as W
from oracle import embed as OE
from oracle import rtn as OR

from gpu_util import dev, host_f16_bits, say

pytestmark = pytest.mark.gpu


def _table(n, k, bits, seed):
    rng = np.random.default_rng(seed)
    w = W.weight(k, n, rng)
    qw = dq.quantize_weight(dev(w), bits, None)
    q, s, z = OR.rtn(w, bits)
    # the table the GPU quantised is the oracle's (codes, scales, zeros)
    assert np.array_equal(dq.wq_unpack(qw.codes, bits, n, k).cpu().numpy(), q)
    assert np.array_equal(host_f16_bits(qw.scales), s.view(np.uint16))
    assert np.array_equal(host_f16_bits(qw.zeros), z.view(np.uint16))
    return qw, q, s, z


def _ids(n, count, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, n, count).astype(np.int32)
    edge = np.array([0, n - 1, -1, n, np.iinfo(np.int32).max, np.iinfo(np.int32).min, 0], dtype=np.int32)
    return np.concatenate([ids, edge, ids[:3]])


def _same_bits(got: torch.Tensor, want: np.ndarray, label):
    g = got.cpu().numpy()
    assert g.dtype == want.dtype
    iv = np.uint16 if want.dtype == np.float16 else np.uint32
    bad = np.nonzero(g.view(iv) != want.view(iv))
    assert bad[0].size == 0, f"{label}: {bad[0].size} outputs differ, first at {bad[0][0]},{bad[1][0]}"


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
@pytest.mark.parametrize("n,k", [(1, 128), (37, 384), (300, 2560), (5, 4224)])
def test_embed_bit_exact(bits, n, k):
    say(f"embed bits={bits} n={n} k={k}")
    qw, q, s, z = _table(n, k, bits, 1000 * bits + n + k)
    ids = _ids(n, 40, n + k)
    idd = torch.from_numpy(ids).cuda()
    for dt, npdt in ((torch.float16, np.float16), (torch.float32, np.float32)):
        got = dq.wq_embed(qw, idd, dt)
        _same_bits(got, OE.embed(q, s, z, ids, npdt), f"bits={bits} n={n} k={k} {npdt.__name__}")


def test_embed_strided_output_and_empty():
    say("embed strided / empty")
    qw, q, s, z = _table(64, 640, 8, 3)
    ids = _ids(64, 9, 4)
    out = torch.full((len(ids), 656), 7.0, dtype=torch.float16, device="cuda")
    dq.wq_embed(qw, torch.from_numpy(ids).cuda(), torch.float16, out=out)
    _same_bits(out[:, :640].contiguous(), OE.embed(q, s, z, ids, np.float16), "strided")
    assert torch.all(out[:, 640:] == 7.0)                 # columns past k untouched
    empty = dq.wq_embed(qw, torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert empty.shape == (0, 640)


def test_embed_head_table_sampled_rows():
    # the 151936 x 2560 int8 head of the int6 block config, as the embedding
    say("embed head table 151936x2560 int8, sampled rows")
    wl = W.WORKLOADS["block_int6_head_int8"]
    idx = len(wl.linears) - 1
    lin = wl.linears[idx]
    w, _, _, _ = W.linear_inputs(0, wl.wid, idx, lin, 1)
    qw = dq.quantize_weight(dev(w), 8, None)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.integers(0, lin.n, 60), [0, lin.n - 1]])).astype(np.int64)
    ids = np.concatenate([rows[::-1], rows[:5]]).astype(np.int32)
    q, s, z = OR.rtn(w[rows], 8)
    del w
    local = np.searchsorted(rows, ids)
    for dt, npdt in ((torch.float16, np.float16), (torch.float32, np.float32)):
        got = dq.wq_embed(qw, torch.from_numpy(ids).cuda(), dt)
        _same_bits(got, OE.embed(q, s, z, local, npdt), f"head {npdt.__name__}")
