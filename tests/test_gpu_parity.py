"""GPU parity: the HIP library against the CPU oracle on small and ragged
shapes (several tiles, partial segments, odd batch sizes), through the C ABI.

Integer work (packing, unpacking, quantised codes, scales and zeros) must
match bit for bit; outputs must meet the tolerance in ``gpu_util``.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_rht_amd as dq
import workloads as W
from oracle import hadamard as OH
from oracle import linear as OL
from oracle import pack as OP
from oracle import rtn as OR

from gpu_util import check_close, dev, dev_u32, host_f16_bits, host_u32, say

pytestmark = pytest.mark.gpu


def _inputs(n, k, m, seed, rht=True, std=0.02):
    rng = np.random.default_rng(seed)
    w = W.weight(k, n, rng, std=std)
    x = W.activations(m, k, rng)
    signs = W.sign_bits(k, rng) if rht else None
    return w, x, signs


# ---------------------------------------------------------------- packing

@pytest.mark.parametrize("bits", [3, 4, 6, 8])
def test_pack_unpack_bit_exact(bits):
    say(f"pack bits={bits}")
    rng = np.random.default_rng(bits)
    n, k = 37, 384
    q = rng.integers(0, 1 << bits, size=(n, k), dtype=np.uint8)
    want = OP.pack(q, bits)
    packed, off = dq.wq_pack(dev(q), bits)
    torch.cuda.synchronize()
    assert off is None
    assert np.array_equal(host_u32(packed).reshape(n, -1), want)
    back = dq.wq_unpack(dev_u32(want.ravel()), bits, n, k)
    assert np.array_equal(back.cpu().numpy(), q)


def test_pack_mixed_bit_exact():
    say("pack mixed")
    rng = np.random.default_rng(7)
    sel = np.array([6, 8, 6, 8], np.uint8)
    n, k = 256, 256
    q = np.concatenate([rng.integers(0, 1 << int(b), size=(64, k), dtype=np.uint8) for b in sel])
    want, want_off = OP.pack_mixed(q, sel)
    packed, off = dq.wq_pack(dev(q), 0, dev(sel))
    torch.cuda.synchronize()
    assert np.array_equal(host_u32(packed), want)
    assert np.array_equal(off.cpu().numpy().astype(np.uint64), want_off)
    back = dq.wq_unpack(dev_u32(want), 0, n, k, dev(sel), off)
    assert np.array_equal(back.cpu().numpy(), q)


# ------------------------------------------------------------- quantiser

@pytest.mark.parametrize("bits", [3, 4, 6, 8])
@pytest.mark.parametrize("rht", [True, False])
def test_quantize_bit_exact(bits, rht):
    say(f"quantize bits={bits} rht={rht}")
    w, _, signs = _inputs(40, 640, 1, 100 + bits, rht)
    w[3, 128:256] = 0.0                      # an all-zero group
    w[5, :128] = np.float32(0.37)            # a constant positive group
    q, s, z = OR.prepare(w, signs, bits)
    qg, sg, zg = dq.wq_quantize(dev(w), bits, dev_u32(signs) if rht else None)
    torch.cuda.synchronize()
    assert np.array_equal(host_f16_bits(sg), s.view(np.uint16))
    assert np.array_equal(host_f16_bits(zg), z.view(np.uint16))
    assert np.array_equal(qg.cpu().numpy(), q)


def test_quantize_mixed_bit_exact():
    say("quantize mixed")
    w, _, signs = _inputs(192, 512, 1, 55)
    sel = np.array([8, 6, 8], np.uint8)
    q, s, z = OR.prepare(w, signs, np.repeat(sel, 64))
    qg, sg, zg = dq.wq_quantize(dev(w), 0, dev_u32(signs), dev(sel))
    torch.cuda.synchronize()
    assert np.array_equal(qg.cpu().numpy(), q)
    assert np.array_equal(host_f16_bits(sg), s.view(np.uint16))
    assert np.array_equal(host_f16_bits(zg), z.view(np.uint16))


# -------------------------------------------------------------- rotation

@pytest.mark.parametrize("m,k", [(1, 128), (5, 1024), (3, 9728)])
def test_rht_apply(m, k):
    say(f"rht m={m} k={k}")
    rng = np.random.default_rng(k + m)
    x = W.activations(m, k, rng)
    signs = W.sign_bits(k, rng)
    ref = OH.rht(x.astype(np.float64), signs)
    y = dq.rht_apply(dev(x), dev_u32(signs)).cpu().numpy().astype(np.float64)
    # one rounding to fp16 of a value computed in fp32: within one fp16 ulp
    ulp = np.maximum(np.abs(ref), 2.0 ** -14) * 2.0 ** -10
    assert np.all(np.abs(y - ref) <= ulp)


def test_rht_apply_in_place_and_strided():
    say("rht in place / strided")
    rng = np.random.default_rng(3)
    m, k, ld = 4, 512, 520
    buf = W.activations(m, ld, rng)
    signs = W.sign_bits(k, rng)
    ref = OH.rht(buf[:, :k].astype(np.float64), signs)
    t = dev(buf)
    view = t[:, :k]
    dq.lib()
    st = dq.lib().rht_apply(view.data_ptr(), view.data_ptr(), dev_u32(signs).data_ptr(), m, k, ld, ld, 128,
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0
    out = t.cpu().numpy()
    ulp = np.maximum(np.abs(ref), 2.0 ** -14) * 2.0 ** -10
    assert np.all(np.abs(out[:, :k].astype(np.float64) - ref) <= ulp)
    assert np.array_equal(out[:, k:], buf[:, k:])      # padding untouched


# ----------------------------------------------------------------- linear

def _gpu_weight(w, signs, bits, sel=None):
    return dq.quantize_weight(dev(w), bits, dev_u32(signs) if signs is not None else None,
                              dev(sel) if sel is not None else None)


def _run_case(n, k, m, bits, rht, out_f32, seed):
    w, x, signs = _inputs(n, k, m, seed, rht)
    q, s, z = OR.prepare(w, signs, bits)
    ref = OL.linear(q, s, z, x, signs)
    qw = _gpu_weight(w, signs, bits)
    y = dq.wq_linear(qw, dev(x), torch.float32 if out_f32 else torch.float16, fuse_rht=rht)
    return check_close(y.float().cpu().numpy(), ref, f"n={n} k={k} m={m} bits={bits}")


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 13, 16])
def test_linear_bits_by_batch(bits, m):
    say(f"linear bits={bits} m={m}")
    _run_case(200, 1024, m, bits, True, False, 1000 * bits + m)


@pytest.mark.parametrize("n,k", [(1, 128), (17, 384), (130, 2560), (64, 9728), (300, 640)])
@pytest.mark.parametrize("rht", [True, False])
@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("m", [1, 3])
def test_linear_shapes(n, k, rht, out_f32, m):
    # m = 1 runs the LDS-ring kernel: odd n leaves a row pair with one row
    say(f"linear n={n} k={k} m={m} rht={rht} f32={out_f32}")
    _run_case(n, k, m, 4, rht, out_f32, n + k + m)


@pytest.mark.parametrize("m", [2, 4, 7, 14])
def test_batch_tiles_k_chunks(m):
    # K = 16384: the arranged activations of a 2-row tile fit in LDS whole,
    # a 4-row tile's (160 KB) in 2 chunks of K, an 8-row tile's in 3; each
    # workgroup walks its units chunk by chunk.  16 rows do not fit even in
    # 4 chunks: m = 14 runs a tile of 8 and one of 6
    say(f"linear K chunks m={m}")
    _run_case(96, 16384, m, 4, True, False, 50 + m)


@pytest.mark.parametrize("k,m", [(16512, 4), (16512, 7), (9856, 16)])
def test_batch_tiles_k_chunks_ragged_tail(k, m):
    # K not a multiple of 512: the last segment holds 4 of 16 slices and
    # falls in the last chunk of K (2, 3 and 3 chunks here)
    say(f"linear K chunks, ragged K={k} m={m}")
    _run_case(96, k, m, 4, True, False, 70 + m)


@pytest.mark.parametrize("m", [4, 7])
def test_batch_tiles_long_k_fall_back(m):
    # K = 65536: a 4-row tile's activations do not fit in LDS even in 4
    # chunks of K: the call falls back to the tiled kernel, which rotates for
    # itself; the result must be the same layer
    say(f"linear long K m={m}")
    _run_case(96, 65536, m, 4, True, False, 55 + m)


@pytest.mark.parametrize("n", [1, 5, 129])
def test_batch_tiles_few_rows(n):
    # fewer row quads than DPP rows: several DPP rows share a quad, one part
    # of K each, and their parts are added in order
    say(f"linear few rows n={n} m=4")
    _run_case(n, 2560, 4, 4, True, False, 60 + n)


@pytest.mark.parametrize("m", [4, 8, 16])
def test_batch_tiles_short_last_workgroup(m):
    # n = 17336 over 256 CUs: 255 workgroups of 68 rows (17 quads, one DPP
    # row each), the last with 64 (16 quads); the last keeps the split of a
    # full workgroup, whose LDS layout the launch sized
    say(f"linear short last workgroup m={m}")
    _run_case(17336, 1024, m, 4, True, False, 80 + m)


@pytest.mark.parametrize("m", [6, 13, 16])
@pytest.mark.parametrize("long_k", [False, True])
def test_batch_tiles_of_eight_and_sixteen(m, long_k):
    # tiles of 8 (m = 6) and 16 (m = 13, 16) batch rows over linears of K
    # 2560, 4096 and 9728 in one call: the activations of 8 rows whole in LDS
    # up to K = 4096 and in 2 chunks at 9728; of 16 rows in 1, 2 and 3 or 4
    shapes = [(256, 2560), (130, 4096)] + ([(64, 9728)] if long_k else [])
    say(f"linear batch tiles m={m} long_k={long_k}")
    qs, xs, refs = [], [], []
    for i, (n, k) in enumerate(shapes):
        w, x, signs = _inputs(n, k, m, 70 + 3 * i + m)
        q, s, z = OR.prepare(w, signs, 3)
        refs.append(OL.linear(q, s, z, x, signs))
        qs.append(_gpu_weight(w, signs, 3))
        xs.append(dev(x))
    for (n, k), y, ref in zip(shapes, dq.wq_linear_batch(qs, xs), refs):
        check_close(y.float().cpu().numpy(), ref, f"batch n={n} k={k} m={m}")


# ---------------------------------------------------------- matrix-core path

@pytest.mark.parametrize("bits", [3, 4, 6, 8])
@pytest.mark.parametrize("m,n,k", [(64, 256, 512), (100, 200, 384), (256, 130, 1024)])
def test_gemm_bits_and_ragged_shapes(bits, m, n, k):
    # M >= 17 runs on MFMA (64 rows: tiles of 64; more: of 128); ragged M and
    # N exercise the partial tiles
    say(f"gemm bits={bits} m={m} n={n} k={k}")
    _run_case(n, k, m, bits, True, False, 7000 + 100 * bits + m)


@pytest.mark.parametrize("out_f32", [False, True])
def test_gemm_split_k_any_n(out_f32):
    # K = 9728 (152 steps of 64) is split over workgroups whose fp32 partial
    # tiles a second pass adds in split order; N = 130 is not a multiple of
    # 4, so that pass adds them one column at a time
    say(f"gemm split-K n=130 k=9728 f32={out_f32}")
    _run_case(130, 9728, 64, 4, True, out_f32, 31 + out_f32)


@pytest.mark.parametrize("rht,out_f32", [(False, False), (True, True), (False, True)])
def test_gemm_rotation_and_output(rht, out_f32):
    say(f"gemm rht={rht} f32={out_f32}")
    _run_case(192, 640, 128, 4, rht, out_f32, 11 + 2 * rht + out_f32)


@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_trained_scales_and_zeros(bits):
    say(f"gemm trained s,z bits={bits}")
    n, k, m = 140, 512, 96
    w, x, signs = _inputs(n, k, m, 300 + bits)
    q, s, z = OR.prepare(w, signs, bits)
    s2, z2 = W.trained_scale_zero(s, z, np.random.default_rng(bits + 1), (1 << bits) - 1)
    ref = OL.linear(q, s2, z2, x, signs)
    packed, _ = dq.wq_pack(dev(q), bits)
    qw = dq.QWeight(bits, n, k, packed, dev(s2), dev(z2), dev_u32(signs))
    check_close(dq.wq_linear(qw, dev(x)).float().cpu().numpy(), ref, "gemm trained s,z")


def test_gemm_mixed_width_runs_on_gemv():
    # the mixed-width layout has no matrix-core kernel: M >= 17 takes the
    # GEMV in chunks and needs no workspace
    say("mixed m=64")
    n, k, m = 192, 512, 64
    w, x, signs = _inputs(n, k, m, 77)
    sel = np.array([8, 6, 8], np.uint8)
    qw = _gpu_weight(w, signs, 0, sel)
    assert dq.wq_linear_workspace(qw, m) == 0
    q, s, z = OR.prepare(w, signs, np.repeat(sel, 64))
    ref = OL.linear(q, s, z, x, signs)
    check_close(dq.wq_linear(qw, dev(x)).float().cpu().numpy(), ref, "mixed m=64")


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
@pytest.mark.parametrize("m", [17, 32, 33, 64])
@pytest.mark.parametrize("k", [640, 9728])
def test_gemm_mid_batch_tiles(bits, m, k):
    # 17..32 rows: tiles of 32 batch rows x 128 outputs; 33..64: 64 x 128.
    # N = 130 leaves a partial last tile (two outputs of a 32-wide block) and
    # K = 9728 is cut over workgroups (split-K partials added afterwards)
    say(f"gemm mid batch bits={bits} m={m} k={k}")
    _run_case(130, k, m, bits, True, k == 9728, 8000 + 10 * bits + m + k)


@pytest.mark.parametrize("m", [17, 29, 40, 63])
def test_linear_mid_batch(m):
    # 17..63 rows: the matrix-core path (narrow tiles of 32 or 64 rows)
    say(f"linear mid batch m={m}")
    _run_case(96, 512, m, 4, True, False, m)
    _run_case(300, 2560, m, 3, True, True, m + 1)


@pytest.mark.parametrize("m", [20, 40, 63])
def test_linear_batch_mid_m_grouped(m):
    # 17..63 rows in one grouped call: every linear's tiles in one
    # matrix-core launch
    say(f"batch mid m={m}")
    shapes = [(256, 2560), (64, 1024), (130, 9728)]
    qs, xs, refs = [], [], []
    for i, (n, k) in enumerate(shapes):
        w, x, signs = _inputs(n, k, m, 140 + i + m)
        q, s_, z = OR.prepare(w, signs, 4)
        refs.append(OL.linear(q, s_, z, x, signs))
        qs.append(_gpu_weight(w, signs, 4))
        xs.append(dev(x))
    for (n, k), y, ref in zip(shapes, dq.wq_linear_batch(qs, xs), refs):
        check_close(y.float().cpu().numpy(), ref, f"batch mid n={n} k={k} m={m}")


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
def test_linear_trained_scales_and_zeros(bits):
    say(f"linear trained s,z bits={bits}")
    n, k, m = 150, 768, 2
    w, x, signs = _inputs(n, k, m, 77 + bits)
    q, s, z = OR.prepare(w, signs, bits)
    s2, z2 = W.trained_scale_zero(s, z, np.random.default_rng(bits), (1 << bits) - 1)
    assert np.any(z2.astype(np.float32) != np.round(z2.astype(np.float32)))
    ref = OL.linear(q, s2, z2, x, signs)
    packed, _ = dq.wq_pack(dev(q), bits)
    qw = dq.QWeight(bits, n, k, packed, dev(s2), dev(z2), dev_u32(signs))
    y = dq.wq_linear(qw, dev(x))
    check_close(y.float().cpu().numpy(), ref, "trained s,z")


@pytest.mark.parametrize("m", [1, 4, 20])
@pytest.mark.parametrize("rht", [True, False])
def test_linear_mixed(m, rht):
    say(f"linear mixed m={m} rht={rht}")
    n, k = 320, 1024
    w, x, signs = _inputs(n, k, m, 900 + m, rht)
    sel = np.array([6, 8, 8, 6, 6], np.uint8)
    q, s, z = OR.prepare(w, signs, np.repeat(sel, 64))
    ref = OL.linear(q, s, z, x, signs)
    qw = _gpu_weight(w, signs, 0, sel)
    y = dq.wq_linear(qw, dev(x), fuse_rht=rht)
    check_close(y.float().cpu().numpy(), ref, "mixed")


def test_mixed_all_six_matches_uniform_six():
    # All-6-bit blocks in the mixed layout hold the same codes, scales and
    # zeros as the uniform int6 layout: the packed words agree bit for bit,
    # and both layouts' products meet the oracle at m = 1 and m = 2.  (The
    # two run different kernels, which sum in different orders, so their
    # outputs are compared through the oracle, not with each other.)
    say("mixed all-6 == int6")
    n, k = 128, 512
    w, x, signs = _inputs(n, k, 2, 31)
    sel = np.array([6, 6], np.uint8)
    mixed, uni = _gpu_weight(w, signs, 0, sel), _gpu_weight(w, signs, 6)
    assert torch.equal(mixed.codes, uni.codes)
    assert torch.equal(mixed.scales, uni.scales) and torch.equal(mixed.zeros, uni.zeros)
    q, s, z = OR.prepare(w, signs, 6)
    for mm in (1, 2):
        ref = OL.linear(q, s, z, x[:mm], signs)
        for qw in (mixed, uni):
            check_close(dq.wq_linear(qw, dev(x[:mm])).float().cpu().numpy(), ref, f"all-6 m={mm}")


def test_batch_call_matches_single_calls():
    say("batch == single")
    shapes = [(256, 2560), (64, 1024), (130, 4096)]
    ws, xs, qs = [], [], []
    for i, (n, k) in enumerate(shapes):
        w, x, signs = _inputs(n, k, 4, 40 + i)
        qs.append(_gpu_weight(w, signs, 4))
        xs.append(dev(x))
    singles = [dq.wq_linear(q, x) for q, x in zip(qs, xs)]
    batch = dq.wq_linear_batch(qs, xs)
    for a, b in zip(singles, batch):
        assert torch.equal(a, b)


@pytest.mark.parametrize("m", [4, 16, 64])
def test_batch_shared_input_rotated_once(m):
    # q, k and v quantised with one sign vector and called on one activation
    # tensor: the call rotates (and arranges) that input once for all three.
    # The outputs equal those of the same call on three copies of the input,
    # bit for bit, and the oracle's within tolerance
    say(f"batch shared input m={m}")
    rng = np.random.default_rng(90 + m)
    signs, signs_o = W.sign_bits(2560, rng), W.sign_bits(4096, rng)
    x, x_o = W.activations(m, 2560, rng), W.activations(m, 4096, rng)
    sg = dev_u32(signs)
    qs, refs = [], []
    for n, k, sb in ((256, 2560, signs), (64, 2560, signs), (64, 2560, signs), (130, 4096, signs_o)):
        w = W.weight(k, n, rng)
        q, s_, z = OR.prepare(w, sb, 4)
        refs.append(OL.linear(q, s_, z, x if k == 2560 else x_o, sb))
        qs.append(dq.quantize_weight(dev(w), 4, sg if k == 2560 else dev_u32(signs_o)))
    xd, xo = dev(x), dev(x_o)
    shared = dq.wq_linear_batch(qs, [xd, xd, xd, xo])
    copies = dq.wq_linear_batch(qs, [xd, xd.clone(), xd.clone(), xo])
    for a, b, ref in zip(shared, copies, refs):
        assert torch.equal(a, b)
        check_close(a.float().cpu().numpy(), ref, f"shared input m={m}")


@pytest.mark.parametrize("m,k", [(16, 9728), (40, 4096)])
def test_deterministic_with_uninitialised_workspace(m, k):
    # the workspace needs no initialisation: one filled with NaN bit
    # patterns gives the same bits as a zeroed one, call after call (16
    # rows at K 9728: the arranged activations of the 16-row tile; 40 rows:
    # the GEMM's rotated activations and K-split partial sums)
    say(f"determinism m={m} k={k}")
    w, x, signs = _inputs(512, k, m, 5)
    qw = _gpu_weight(w, signs, 4)
    need = dq.wq_linear_workspace(qw, m)
    assert need > 0
    xd = dev(x)
    first = dq.wq_linear(qw, xd, workspace=dq.new_workspace(need))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for _ in range(5):
        assert torch.equal(dq.wq_linear(qw, xd, workspace=ws), first)


@pytest.mark.parametrize("m", [24, 63])
def test_split_k_sums_stable(m):
    # 17..64 rows: K = 9728 and 4096 are cut over workgroups whose partials
    # a second kernel adds.  Back-to-back calls on one workspace, no host
    # sync between them, must give the same bits every time and match the
    # oracle; a call on the caller's rotated input (natural order instead of
    # the rotation's pair order) must match it too.
    say(f"split-K sums m={m}")
    shapes = [(2560, 9728), (640, 4096), (130, 2560)]
    qs, xs, xrot, refs = [], [], [], []
    for i, (n, k) in enumerate(shapes):
        w, x, signs = _inputs(n, k, m, 900 + 10 * m + i)
        q, s_, z = OR.prepare(w, signs, 4)
        refs.append(OL.linear(q, s_, z, x, signs))
        qs.append(_gpu_weight(w, signs, 4))
        xs.append(dev(x))
        xrot.append(dq.rht_apply(dev(x), dev_u32(signs)))
    ws = dq.new_workspace(dq.wq_linear_batch_workspace(qs, m))
    outs = [dq.wq_linear_batch(qs, xs, workspace=ws) for _ in range(20)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert torch.equal(a, b)
    for (n, k), y, ref in zip(shapes, outs[0], refs):
        check_close(y.float().cpu().numpy(), ref, f"split sums n={n} k={k} m={m}")
    for (n, k), y, ref in zip(shapes, dq.wq_linear_batch(qs, xrot, fuse_rht=False), refs):
        check_close(y.float().cpu().numpy(), ref, f"split sums, rotated by the caller n={n} k={k} m={m}")


def test_graph_replay_matches_eager():
    say("graph replay")
    w, x, signs = _inputs(384, 2560, 1, 6)
    qw = _gpu_weight(w, signs, 4)
    xd = dev(x)
    ws = dq.new_workspace(dq.wq_linear_workspace(qw, 1))
    eager = dq.wq_linear(qw, xd, workspace=ws)
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dq.wq_linear(qw, xd, workspace=ws, out=out)   # warm up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dq.wq_linear(qw, xd, workspace=ws, out=out)
    for _ in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        assert torch.equal(dq.wq_linear(qw, xd, workspace=ws), eager)
