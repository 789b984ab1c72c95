"""Property tests (hypothesis) over code width, K, N and M (CPU only).

* The oracle's packer: every code matrix survives pack -> unpack; a single
  flipped bit of one code flips exactly one bit of the packed words, at the
  place the layout in ``oracle/pack.py`` gives (rows contiguous along K, runs
  of 32/8/16/4 codes in 3/1/3/1 words, code j of a run at bit bits*j of the
  run's little-endian integer); mixed-width blocks sit at their offsets.
* The C ABI's host side: the library's word counts agree with the oracle's
  layout for every width and K; a single linear's workspace equals that of a
  group of one; a group's workspace is the sum of its members' (batch
  tiles) or holds every member's rotated activations (matrix cores); and a
  call with any one defect is refused with that defect's status before any
  HIP call (no GPU is touched here); a mixed layout's host copy of its
  widths is checked value by value on the host.
"""

import ctypes

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import dequant_gemv_rht_amd as dq
from oracle import pack as P

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])

bits_st = st.sampled_from([3, 4, 6, 8])
k_st = st.integers(1, 8).map(lambda i: 128 * i)
n_st = st.integers(1, 200)
m_st = st.integers(1, 16)
RUN = {3: (32, 3), 4: (8, 1), 6: (16, 3), 8: (4, 1)}   # codes per run, words per run


def _codes(rng, n, k, bits):
    return rng.integers(0, 1 << bits, size=(n, k), dtype=np.uint8)


@SETTINGS
@given(bits=bits_st, k=k_st, n=st.integers(1, 24), seed=st.integers(0, 2**32 - 1))
def test_oracle_pack_round_trip(bits, k, n, seed):
    q = _codes(np.random.default_rng(seed), n, k, bits)
    words = P.pack(q, bits)
    assert words.shape == (n, k * bits // 32)
    assert np.array_equal(P.unpack(words, bits, n, k), q)


@SETTINGS
@given(bits=bits_st, k=k_st, seed=st.integers(0, 2**32 - 1), data=st.data())
def test_oracle_pack_single_bit_locality(bits, k, seed, data):
    n = 3
    q = _codes(np.random.default_rng(seed), n, k, bits)
    r = data.draw(st.integers(0, n - 1))
    c = data.draw(st.integers(0, k - 1))
    t = data.draw(st.integers(0, bits - 1))
    q2 = q.copy()
    q2[r, c] ^= np.uint8(1 << t)
    diff = P.pack(q, bits) ^ P.pack(q2, bits)
    per_run, wpr = RUN[bits]
    pos = (c % per_run) * bits + t                       # bit within the run's integer
    word = r * (k * bits // 32) + (c // per_run) * wpr + pos // 32
    flat = diff.reshape(-1)
    assert np.count_nonzero(flat) == 1
    assert int(flat[word]) == 1 << (pos % 32)


@SETTINGS
@given(k=k_st, sel=st.lists(st.sampled_from([6, 8]), min_size=1, max_size=4), seed=st.integers(0, 2**32 - 1))
def test_oracle_mixed_blocks_at_their_offsets(k, sel, seed):
    sel = np.array(sel, np.uint8)
    n = 64 * len(sel)
    rng = np.random.default_rng(seed)
    q = np.concatenate([_codes(rng, 64, k, int(b)) for b in sel])
    words, off = P.pack_mixed(q, sel)
    assert off[0] == 0 and len(words) == int(off[-1])
    for i, b in enumerate(sel):
        assert int(off[i + 1] - off[i]) == 64 * k * int(b) // 32
        block = words[int(off[i]):int(off[i + 1])].reshape(64, -1)
        assert np.array_equal(block, P.pack(q[64 * i:64 * (i + 1)], int(b)))
    assert np.array_equal(P.unpack_mixed(words, sel, n, k), q)


# ---------------------------------------------------------------------------
# The C ABI, host side only


@pytest.fixture(scope="module")
def lib():
    return dq.lib()


def _weight(bits=4, n=64, k=256, rht=False, **kw):
    base = dict(bits=bits, group=128, n=n, k=k, codes=16, scales=16, zeros=16, block_bits=None,
                block_off=None, rht_signs=16 if rht else None, rht_block=128 if rht else 0)
    base.update(kw)
    return dq.WqWeight(**base)


@SETTINGS
@given(bits=bits_st, k=k_st, n=n_st)
def test_abi_packed_words_match_oracle_layout(lib, bits, k, n):
    assert lib.wq_packed_words(bits, n, k, None) == n * P.words_per_row(bits, k)


@SETTINGS
@given(k=k_st, sel=st.lists(st.sampled_from([6, 8]), min_size=1, max_size=6))
def test_abi_mixed_packed_words_match_oracle_offsets(lib, k, sel):
    arr = (ctypes.c_uint8 * len(sel))(*sel)
    assert lib.wq_packed_words(0, 64 * len(sel), k, arr) == int(P.block_offsets(np.array(sel), k)[-1])


@SETTINGS
@given(bits=bits_st, k=k_st, n=n_st, m=st.integers(1, 600), rht=st.booleans())
def test_abi_single_workspace_is_a_group_of_one(lib, bits, k, n, m, rht):
    w = _weight(bits, n, k, rht)
    one = (dq.WqWeight * 1)(w)
    assert lib.wq_linear_workspace(ctypes.byref(w), m) == lib.wq_linear_batch_workspace(1, one, m)


@SETTINGS
@given(bits=bits_st, shapes=st.lists(st.tuples(n_st, k_st), min_size=1, max_size=8), m=st.integers(2, 600),
       rht=st.booleans())
def test_abi_group_workspace(lib, bits, shapes, m, rht):
    ws = [_weight(bits, n, k, rht) for n, k in shapes]
    arr = (dq.WqWeight * len(ws))(*ws)
    total = lib.wq_linear_batch_workspace(len(ws), arr, m)
    singles = [lib.wq_linear_workspace(ctypes.byref(w), m) for w in ws]
    if m <= 16:
        # batch tiles: each linear's arranged activations, side by side
        assert total == sum(singles)
    else:
        # matrix cores: every linear's rotated activations, fp16 [m][k]
        if rht:
            assert total >= sum(m * k * 2 for _, k in shapes)
        assert total >= max(singles)   # a group never needs less than its largest member


DEFECTS = {
    # weight descriptor
    "bits": (dict(bits=5), dq.WQ_E_UNSUPPORTED),
    "group": (dict(group=64), dq.WQ_E_UNSUPPORTED),
    "k not a multiple of 128": (dict(k_off=64), dq.WQ_E_ARG),
    "n zero": (dict(n=0), dq.WQ_E_ARG),
    "codes NULL": (dict(codes=None), dq.WQ_E_ARG),
    "scales misaligned": (dict(scales=24), dq.WQ_E_ALIGN),
    "mixed n": (dict(bits=0, n_off=32), dq.WQ_E_ARG),
    "mixed tables": (dict(bits=0), dq.WQ_E_ARG),
    "rht block": (dict(rht_block=64), dq.WQ_E_UNSUPPORTED),
    # activations / outputs
    "m zero": (dict(m=0), dq.WQ_E_ARG),
    "x NULL": (dict(x=None), dq.WQ_E_ARG),
    "x misaligned": (dict(x=24), dq.WQ_E_ALIGN),
    "ldx short": (dict(ldx_off=-8), dq.WQ_E_ARG),
    "ldx odd": (dict(ldx_off=4), dq.WQ_E_ALIGN),
    "ldy short": (dict(ldy_off=-1), dq.WQ_E_ARG),
    "y dtype": (dict(ydt=9), dq.WQ_E_ARG),
    "flags": (dict(flags=4), dq.WQ_E_ARG),
}


@SETTINGS
@given(bits=bits_st, k=k_st, n=st.integers(1, 4).map(lambda i: 64 * i), m=m_st,
       defect=st.sampled_from(sorted(DEFECTS)))
def test_abi_any_single_defect_is_refused(lib, bits, k, n, m, defect):
    kw, status = DEFECTS[defect]
    kw = dict(kw)
    wk = dict(bits=kw.pop("bits", bits), n=kw.pop("n", n) + kw.pop("n_off", 0), k=k + kw.pop("k_off", 0),
              rht="rht_block" in kw)
    for f in ("group", "codes", "scales", "rht_block"):
        if f in kw:
            wk[f] = kw.pop(f)
    w = _weight(**wk)
    a = dict(m=m, x=16, ldx=k, y=16, ydt=dq.WQ_F16, ldy=n, flags=0)
    a["ldx"] += kw.pop("ldx_off", 0)
    a["ldy"] += kw.pop("ldy_off", 0)
    a.update(kw)
    st_ = lib.wq_linear(ctypes.byref(w), a["x"], a["m"], a["ldx"], a["y"], a["ydt"], a["ldy"], a["flags"],
                        16, 1 << 40, None)
    assert st_ == status, (defect, lib.wq_last_error())
    assert lib.wq_last_error().decode()


@SETTINGS
@given(k=k_st, widths=st.lists(st.integers(0, 255), min_size=1, max_size=12), data=st.data())
def test_abi_host_widths_checked_on_the_host(lib, k, widths, data):
    # a mixed layout's optional host copy of its widths: any value other than
    # 6 and 8 is refused (WQ_E_ARG, naming the first bad block) before any HIP
    # call; valid widths pass the weight checks and the call meets its next
    # defect, the output type (so nothing is launched either way)
    if data.draw(st.booleans()):
        widths = [data.draw(st.sampled_from([6, 8])) for _ in widths]
    arr = (ctypes.c_uint8 * len(widths))(*widths)
    w = _weight(bits=0, n=64 * len(widths), k=k, block_bits=16, block_off=16,
                block_bits_host=ctypes.addressof(arr))
    st_ = lib.wq_linear(ctypes.byref(w), 16, 1, k, 16, 9, 64 * len(widths), 0, 16, 1 << 40, None)
    msg = lib.wq_last_error().decode()
    bad = [i for i, v in enumerate(widths) if v not in (6, 8)]
    assert st_ == dq.WQ_E_ARG
    if bad:
        assert f"block_bits_host[{bad[0]}]={widths[bad[0]]}" in msg, msg
    else:
        assert "y_dtype" in msg, msg
