"""Python binding of libwq (the rotated grouped-affine low-bit linear layer).

Argument marshalling only: every step runs in the HIP kernels of
``_lib/libwq.so``, built for gfx950 by ``dequant_gemv_rht_amd.build``.
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: if the library is missing, importing the functions raises.

Functions mirror the C ABI in ``include/wq.h``:

  wq_quantize(w, bits, signs=None, block_bits=None)  -> (codes, scales, zeros)
  wq_pack(codes, bits, block_bits=None)              -> QWeight pieces (packed, block_off)
  wq_unpack(packed, bits, n, k, block_bits=None, block_off=None) -> codes
  rht_apply(x, signs, out=None)                      -> rotated fp16 activations
  wq_linear(weight, x, out_dtype=float16, fuse_rht=True, workspace=None) -> y
  wq_linear_batch(weights, xs, out_dtypes=None, fuse_rht=True, workspace=None) -> [y]
  wq_linear_batch_noalloc(weights, xs, out_dtypes=None, fuse_rht=True, out=None) -> [y]
  wq_embed(table, ids, out_dtype=float16, out=None)  -> dequantised table rows
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libwq.so")

WQ_OK, WQ_E_ARG, WQ_E_UNSUPPORTED, WQ_E_ALIGN, WQ_E_WORKSPACE, WQ_E_HIP = 0, -1, -2, -3, -4, -5
WQ_F16, WQ_F32 = 1, 2
WQ_FUSE_RHT = 1
WQ_MAX_BATCH = 8
STATUS_NAMES = {0: "WQ_OK", -1: "WQ_E_ARG", -2: "WQ_E_UNSUPPORTED", -3: "WQ_E_ALIGN",
                -4: "WQ_E_WORKSPACE", -5: "WQ_E_HIP"}

# Every function the header declares, with its ctypes signature.
_vp, _i32, _i64, _u32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t


class WqWeight(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("codes", _vp), ("scales", _vp), ("zeros", _vp),
                ("block_bits", _vp), ("block_off", _vp),
                ("rht_signs", _vp), ("rht_block", ctypes.c_int32),
                ("block_bits_host", _vp)]


SIGNATURES = {
    "wq_packed_words": (_sz, [_i32, _i64, _i64, _vp]),
    "wq_quantize": (_i32, [_i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "wq_pack": (_i32, [_i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "wq_unpack": (_i32, [_i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "rht_apply": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp]),
    "wq_linear_workspace": (_sz, [ctypes.POINTER(WqWeight), _i64]),
    "wq_linear": (_i32, [ctypes.POINTER(WqWeight), _vp, _i64, _i64, _vp, _i32, _i64, _u32, _vp, _sz, _vp]),
    "wq_linear_batch_workspace": (_sz, [_i32, ctypes.POINTER(WqWeight), _i64]),
    "wq_linear_batch": (_i32, [_i32, ctypes.POINTER(WqWeight), ctypes.POINTER(_vp), ctypes.POINTER(_i64),
                               _i64, ctypes.POINTER(_vp), ctypes.POINTER(_i32), ctypes.POINTER(_i64),
                               _u32, _vp, _sz, _vp]),
    "wq_last_error": (ctypes.c_char_p, []),
    "wq_stream_read": (_i32, [_vp, _sz, _vp, _vp]),
    "wq_embed": (_i32, [ctypes.POINTER(WqWeight), _vp, _i64, _vp, _i32, _i64, _vp]),
    "wq_linear_batch_noalloc": (_i32, [_i32, ctypes.POINTER(WqWeight), ctypes.POINTER(_vp),
                                       ctypes.POINTER(_i64), _i64, ctypes.POINTER(_vp), ctypes.POINTER(_i32),
                                       ctypes.POINTER(_i64), _u32, _vp]),
}
NOALLOC_SCRATCH_BYTES = 64 << 20   # WQ_NOALLOC_SCRATCH_BYTES

_lib = None


class WqError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def lib():
    """The loaded libwq (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libwq is not built ({LIB_PATH} missing): run "
                               f"`python -m dequant_gemv_rht_amd.build` (hipcc, gfx950)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(fn: str, status: int):
    if status != WQ_OK:
        raise WqError(fn, status, lib().wq_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


@dataclass
class QWeight:
    """A quantised weight on the GPU in libwq's layout."""
    bits: int                     # 3, 4, 6, 8, or 0 for mixed 6/8
    n: int
    k: int
    codes: torch.Tensor           # int32 view of the packed uint32 words
    scales: torch.Tensor          # float16 [n][k/128]
    zeros: torch.Tensor           # float16 [n][k/128]
    signs: Optional[torch.Tensor] = None       # int32 view of uint32 [k/32]
    block_bits: Optional[torch.Tensor] = None  # uint8 [n/64]
    block_off: Optional[torch.Tensor] = None   # int64 view of uint64 [n/64 + 1]
    # mixed width: also hand the library a host copy of block_bits (made
    # once, here), so the batch-1 kernel need not read the block table first
    host_widths: bool = True

    def __post_init__(self):
        self._bits_host = None
        if self.bits == 0 and self.block_bits is not None and self.host_widths:
            self._bits_host = np.ascontiguousarray(self.block_bits.cpu().numpy(), dtype=np.uint8)

    def c_struct(self) -> WqWeight:
        bh = self._bits_host.ctypes.data if self._bits_host is not None else None
        return WqWeight(self.bits, 128, self.n, self.k, _ptr(self.codes), _ptr(self.scales),
                        _ptr(self.zeros), _ptr(self.block_bits), _ptr(self.block_off),
                        _ptr(self.signs), 128 if self.signs is not None else 0, bh)


def wq_packed_words(bits: int, n: int, k: int, block_bits_host=None) -> int:
    bb = None
    if block_bits_host is not None:
        import numpy as np
        arr = np.ascontiguousarray(np.asarray(block_bits_host, dtype=np.uint8))
        bb = arr.ctypes.data
        words = lib().wq_packed_words(bits, n, k, bb)
    else:
        words = lib().wq_packed_words(bits, n, k, None)
    if words == 0:
        raise WqError("wq_packed_words", WQ_E_ARG, lib().wq_last_error().decode())
    return words


def wq_quantize(w: torch.Tensor, bits: int, signs: Optional[torch.Tensor] = None,
                block_bits: Optional[torch.Tensor] = None):
    """Rotate (if signs) and round-to-nearest quantise fp32 [n][k] -> (codes u8, scales f16, zeros f16)."""
    _dev(w, torch.float32, "w")
    n, k = w.shape
    codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // 128), dtype=torch.float16, device=w.device)
    zeros = torch.empty((n, k // 128), dtype=torch.float16, device=w.device)
    _check("wq_quantize", lib().wq_quantize(bits, n, k, _ptr(w), _ptr(signs), _ptr(block_bits),
                                            _ptr(codes), _ptr(scales), _ptr(zeros), _stream()))
    return codes, scales, zeros


def wq_pack(codes: torch.Tensor, bits: int, block_bits: Optional[torch.Tensor] = None):
    """Pack uint8 [n][k] codes; returns (packed int32 words, block_off int64 or None)."""
    _dev(codes, torch.uint8, "codes")
    n, k = codes.shape
    bb_host = None if block_bits is None else block_bits.cpu().numpy()
    words = wq_packed_words(bits, n, k, bb_host)
    packed = torch.empty(words, dtype=torch.int32, device=codes.device)
    block_off = None
    if bits == 0:
        block_off = torch.empty(n // 64 + 1, dtype=torch.int64, device=codes.device)
    _check("wq_pack", lib().wq_pack(bits, n, k, _ptr(codes), _ptr(block_bits), _ptr(packed),
                                    _ptr(block_off), _stream()))
    return packed, block_off


def wq_unpack(packed: torch.Tensor, bits: int, n: int, k: int, block_bits=None, block_off=None):
    codes = torch.empty((n, k), dtype=torch.uint8, device=packed.device)
    _check("wq_unpack", lib().wq_unpack(bits, n, k, _ptr(packed), _ptr(block_bits), _ptr(block_off),
                                        _ptr(codes), _stream()))
    return codes


def rht_apply(x: torch.Tensor, signs: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Block-128 random Hadamard rotation of fp16 [m][k] activations."""
    _dev(x, torch.float16, "x")
    m, k = x.shape
    y = torch.empty_like(x) if out is None else out
    _check("rht_apply", lib().rht_apply(_ptr(x), _ptr(y), _ptr(signs), m, k, x.stride(0), y.stride(0),
                                        128, _stream()))
    return y


def quantize_weight(w: torch.Tensor, bits: int, signs: Optional[torch.Tensor] = None,
                    block_bits: Optional[torch.Tensor] = None) -> QWeight:
    """wq_quantize + wq_pack into a QWeight."""
    codes, scales, zeros = wq_quantize(w, bits, signs, block_bits)
    packed, block_off = wq_pack(codes, bits, block_bits)
    n, k = w.shape
    return QWeight(bits, n, k, packed, scales, zeros, signs, block_bits, block_off)


def wq_linear_workspace(weight: QWeight, m: int) -> int:
    st = weight.c_struct()
    size = lib().wq_linear_workspace(ctypes.byref(st), m)
    if size == ctypes.c_size_t(-1).value:
        raise WqError("wq_linear_workspace", WQ_E_ARG, lib().wq_last_error().decode())
    return size


def new_workspace(size: int, device="cuda") -> torch.Tensor:
    """A workspace of ``size`` bytes (zero-filled; the library needs no particular contents)."""
    return torch.zeros(max(size, 16), dtype=torch.uint8, device=device)


def wq_linear(weight: QWeight, x: torch.Tensor, out_dtype=torch.float16, fuse_rht: bool = True,
              workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    _dev(x, torch.float16, "x")
    m = x.shape[0]
    ydt = WQ_F32 if out_dtype == torch.float32 else WQ_F16
    y = torch.empty((m, weight.n), dtype=out_dtype, device=x.device) if out is None else out
    need = wq_linear_workspace(weight, m)
    if workspace is None:
        workspace = new_workspace(need, x.device)
    st = weight.c_struct()
    _check("wq_linear", lib().wq_linear(ctypes.byref(st), _ptr(x), m, x.stride(0), _ptr(y), ydt,
                                        y.stride(0), WQ_FUSE_RHT if fuse_rht else 0, _ptr(workspace),
                                        workspace.numel(), _stream()))
    return y


def wq_linear_batch_workspace(weights: Sequence[QWeight], m: int) -> int:
    arr = (WqWeight * len(weights))(*[w.c_struct() for w in weights])
    size = lib().wq_linear_batch_workspace(len(weights), arr, m)
    if size == ctypes.c_size_t(-1).value:
        raise WqError("wq_linear_batch_workspace", WQ_E_ARG, lib().wq_last_error().decode())
    return size


class BatchCall:
    """Pre-marshalled arguments of one wq_linear_batch call (reusable)."""

    def __init__(self, weights: Sequence[QWeight], xs: Sequence[torch.Tensor], ys: Sequence[torch.Tensor],
                 fuse_rht: bool, workspace: torch.Tensor):
        c = len(weights)
        self.count = c
        self.m = xs[0].shape[0]
        self.w = (WqWeight * c)(*[w.c_struct() for w in weights])
        self.x = (_vp * c)(*[x.data_ptr() for x in xs])
        self.ldx = (_i64 * c)(*[x.stride(0) for x in xs])
        self.y = (_vp * c)(*[y.data_ptr() for y in ys])
        self.ydt = (_i32 * c)(*[WQ_F32 if y.dtype == torch.float32 else WQ_F16 for y in ys])
        self.ldy = (_i64 * c)(*[y.stride(0) for y in ys])
        self.flags = WQ_FUSE_RHT if fuse_rht else 0
        self.ws = workspace
        self._keep = (list(weights), list(xs), list(ys))

    def __call__(self, stream: Optional[int] = None):
        _check("wq_linear_batch", lib().wq_linear_batch(
            self.count, self.w, self.x, self.ldx, self.m, self.y, self.ydt, self.ldy, self.flags,
            self.ws.data_ptr(), self.ws.numel(), _stream() if stream is None else stream))


def wq_linear_batch(weights: Sequence[QWeight], xs: Sequence[torch.Tensor], out_dtypes=None,
                    fuse_rht: bool = True, workspace: Optional[torch.Tensor] = None):
    m = xs[0].shape[0]
    out_dtypes = out_dtypes or [torch.float16] * len(weights)
    ys = [torch.empty((m, w.n), dtype=dt, device=xs[0].device) for w, dt in zip(weights, out_dtypes)]
    if workspace is None:
        workspace = new_workspace(wq_linear_batch_workspace(weights, m), xs[0].device)
    BatchCall(weights, xs, ys, fuse_rht, workspace)()
    return ys


def wq_linear_batch_noalloc(weights: Sequence[QWeight], xs: Sequence[torch.Tensor], out_dtypes=None,
                            fuse_rht: bool = True, out: Optional[Sequence[torch.Tensor]] = None):
    """wq_linear_batch on the library's static scratch: no workspace argument,
    and the call allocates no device memory (outputs are allocated here
    unless given in ``out``)."""
    m = xs[0].shape[0]
    out_dtypes = out_dtypes or [torch.float16] * len(weights)
    ys = list(out) if out is not None else [torch.empty((m, w.n), dtype=dt, device=xs[0].device)
                                            for w, dt in zip(weights, out_dtypes)]
    c = len(weights)
    _check("wq_linear_batch_noalloc", lib().wq_linear_batch_noalloc(
        c, (WqWeight * c)(*[w.c_struct() for w in weights]), (_vp * c)(*[x.data_ptr() for x in xs]),
        (_i64 * c)(*[x.stride(0) for x in xs]), m, (_vp * c)(*[y.data_ptr() for y in ys]),
        (_i32 * c)(*[WQ_F32 if y.dtype == torch.float32 else WQ_F16 for y in ys]),
        (_i64 * c)(*[y.stride(0) for y in ys]), WQ_FUSE_RHT if fuse_rht else 0, _stream()))
    return ys


def wq_embed(table: QWeight, ids: torch.Tensor, out_dtype=torch.float16, out: Optional[torch.Tensor] = None):
    """Rows ``ids`` of the quantised ``table``, dequantised: [len(ids)][k]."""
    _dev(ids, torch.int32, "ids")
    count = ids.numel()
    y = torch.empty((count, table.k), dtype=out_dtype, device=ids.device) if out is None else out
    st = table.c_struct()
    _check("wq_embed", lib().wq_embed(ctypes.byref(st), _ptr(ids), count, _ptr(y),
                                      WQ_F32 if out_dtype == torch.float32 else WQ_F16,
                                      y.stride(0) if count else table.k, _stream()))
    return y


def stream_read(src: torch.Tensor, sink: torch.Tensor, nbytes: Optional[int] = None) -> None:
    """Plain streaming read of ``nbytes`` (default: all) of ``src`` on the
    current stream: the read ceiling a workload's weight stream is compared
    with (include/wq_measure.h)."""
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    if not src.is_cuda or not sink.is_cuda or sink.numel() * sink.element_size() < 4:
        raise ValueError("stream_read: src and a 4-byte sink must be GPU tensors")
    _check("wq_stream_read", lib().wq_stream_read(src.data_ptr(), n, sink.data_ptr(), _stream()))
