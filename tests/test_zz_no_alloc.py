"""wq_linear_batch_noalloc, the grouped call on the library's static scratch:
its outputs equal those of wq_linear_batch with a caller's workspace bit for
bit (the same kernels, launched the same way) and meet the oracle's
tolerance, on consecutive calls whose second is smaller than the first (the
scratch keeps the previous call's contents, which must not matter)."""

import numpy as np
import pytest
import torch

import dequant_gemv_rht_amd as dq
import workloads as W
from oracle import linear as OL
from oracle import rtn as OR

from gpu_util import check_close, dev, dev_u32, say

pytestmark = pytest.mark.gpu

# K = 9728 is split over workgroups at 64 rows and more (partial sums in the
# workspace); below 64 rows the workspace holds the arranged activations
SHAPES = [(256, 2560), (130, 9728), (64, 1024)]


def _linears(m, seed, bits=4):
    qs, xs, refs = [], [], []
    for i, (n, k) in enumerate(SHAPES):
        rng = np.random.default_rng(seed + i)
        w = W.weight(k, n, rng)
        x = W.activations(m, k, rng)
        signs = W.sign_bits(k, rng)
        q, s, z = OR.prepare(w, signs, bits)
        refs.append(OL.linear(q, s, z, x, signs))
        qs.append(dq.quantize_weight(dev(w), bits, dev_u32(signs)))
        xs.append(dev(x))
    return qs, xs, refs


@pytest.mark.parametrize("ms", [(96, 16), (16, 4), (4, 1)], ids=["96-then-16", "16-then-4", "4-then-1"])
def test_noalloc_matches_workspace_call(ms):
    for m in ms:
        say(f"noalloc grouped call m={m}")
        qs, xs, refs = _linears(m, 300 + m)
        assert 0 < dq.wq_linear_batch_workspace(qs, m) <= dq.NOALLOC_SCRATCH_BYTES or m == 1
        want = dq.wq_linear_batch(qs, xs)
        got = dq.wq_linear_batch_noalloc(qs, xs)
        torch.cuda.synchronize()
        for (n, k), a, b, ref in zip(SHAPES, got, want, refs):
            assert torch.equal(a, b), f"noalloc differs from the workspace call: n={n} k={k} m={m}"
            rel, mx = check_close(a.float().cpu().numpy(), ref, f"noalloc n={n} k={k} m={m}")
            say(f"  n={n} k={k}: rel-L2 {rel:.2e} max/rms {mx:.2e}")


def test_noalloc_rejects_calls_beyond_the_scratch():
    # 4096 rows of K = 9728 need 80 MB of rotated activations: refused before
    # anything is launched, with the sizes in the message
    say("noalloc: a call beyond the scratch")
    qs, xs, _ = _linears(4, 7)
    x_big = torch.zeros((4096, 9728), dtype=torch.float16, device="cuda")
    with pytest.raises(dq.WqError) as e:
        dq.wq_linear_batch_noalloc([qs[1]], [x_big])
    assert e.value.status == dq.WQ_E_WORKSPACE
    assert "static scratch" in str(e.value)
