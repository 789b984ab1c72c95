"""Seeded synthetic inputs for the grouped-affine low-bit linear layer.

This module only draws random numbers. It holds no step of the method itself:
no rotation, no quantisation, no packing, no dequantisation and no product.
The CPU oracle and the HIP path both take their inputs from here, so the
two never exchange data except through these arrays.

Every array comes from ``numpy.random.default_rng`` seeded with
``SeedSequence([seed, workload_id, tensor_id])`` (PCG64), so a given
(seed, workload, tensor) triple yields the same bytes on every machine.

Recipe (the model cards describe a 4B-class decoder; no trained weights or
calibration data are available, so these stand in for them):

* weights: fp32 ``0.02 * N(0, 1)``, shape ``[N][K]`` (output rows, input
  channels); ``round(0.01 * K)`` input channels, chosen without replacement,
  are multiplied by 20 to act as outlier channels;
* activations: fp16 ``N(0, 1)``, shape ``[M][K]`` (rounded to nearest even);
* rotation signs: ``K`` independent fair bits packed 32 to a ``uint32`` word,
  bit ``k & 31`` of word ``k >> 5`` belongs to input channel ``k``; a set bit
  means a sign of -1;
* mixed-width selectors: one byte per 64-row output block holding the bit
  width (6 or 8); exactly ``round(0.2 * blocks)`` blocks, chosen without
  replacement, are 8-bit.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GROUP = 128          # quantisation group along K (also the rotation block)
MIXED_ROWS = 64      # output rows per mixed-width block

# The seven projections of one 4B-class decoder block: (name, K, N) with
# K the input (reduction) width and N the number of output rows.
PROJECTIONS = (
    ("q_proj", 2560, 4096),
    ("k_proj", 2560, 1024),
    ("v_proj", 2560, 1024),
    ("o_proj", 4096, 2560),
    ("gate_proj", 2560, 9728),
    ("up_proj", 2560, 9728),
    ("down_proj", 9728, 2560),
)
# Tied embedding / output head of the same model family: 151936 x 2560.
HEAD = ("lm_head", 2560, 151936)


def rng_for(seed: int, workload_id: int, tensor_id: int) -> np.random.Generator:
    """Independent PCG64 stream for one tensor of one workload."""
    return np.random.default_rng(np.random.SeedSequence([seed, workload_id, tensor_id]))


def weight(k: int, n: int, rng: np.random.Generator, std: float = 0.02,
           outlier_frac: float = 0.01, outlier_scale: float = 20.0) -> np.ndarray:
    """fp32 [n][k] weight with ``round(outlier_frac*k)`` scaled input channels."""
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    n_out = int(round(outlier_frac * k))
    if n_out:
        idx = rng.choice(k, n_out, replace=False)
        w[:, idx] *= np.float32(outlier_scale)
    return w


def activations(m: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """fp16 [m][k] activations drawn from N(0, 1)."""
    return rng.standard_normal((m, k)).astype(np.float16)


def scaled_activations(m: int, k: int, rng: np.random.Generator, rms, outlier_frac: float = 0.0,
                       outlier_scale: float = 1.0) -> np.ndarray:
    """fp16 [m][k] activations ``rms * N(0, 1)`` (``rms`` a number, or one per
    batch row), with ``round(outlier_frac * k)`` input channels, chosen without
    replacement, multiplied by ``outlier_scale``.  Rounded to fp16 once, after
    scaling, so small values may be fp16 subnormals, as they would be in a
    real fp16 activation tensor."""
    x = rng.standard_normal((m, k))
    x *= np.broadcast_to(np.asarray(rms, dtype=np.float64).reshape(-1, 1), (m, 1))
    n_out = int(round(outlier_frac * k))
    if n_out:
        x[:, rng.choice(k, n_out, replace=False)] *= outlier_scale
    return x.astype(np.float16)


def sign_bits(k: int, rng: np.random.Generator) -> np.ndarray:
    """``k`` random sign bits packed into ``uint32 [k/32]`` (bit set => -1)."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    return rng.integers(0, 1 << 32, size=k // 32, dtype=np.uint64).astype(np.uint32)


def block_selector(n: int, rng: np.random.Generator, frac8: float = 0.2) -> np.ndarray:
    """``uint8 [n/64]`` widths: exactly ``round(frac8 * blocks)`` are 8, the rest 6."""
    if n % MIXED_ROWS:
        raise ValueError("n must be a multiple of 64")
    nb = n // MIXED_ROWS
    sel = np.full(nb, 6, dtype=np.uint8)
    sel[rng.choice(nb, int(round(frac8 * nb)), replace=False)] = 8
    return sel


def trained_scale_zero(s16: np.ndarray, z16: np.ndarray, rng: np.random.Generator,
                       qmax) -> tuple[np.ndarray, np.ndarray]:
    """Scales and zeros moved off their round-to-nearest values.

    Stands in for scales and zero points that were trained after
    quantisation: the codes keep their format, but a scale may be any
    positive fp16 value and a zero point any fp16 value, not only an integer.
    Scales are multiplied by a factor in [0.9, 1.1]; zeros get a uniform
    offset in [-0.5, 0.5] and stay within [0, qmax].
    """
    s = s16.astype(np.float32) * rng.uniform(0.9, 1.1, size=s16.shape).astype(np.float32)
    z = z16.astype(np.float32) + rng.uniform(-0.5, 0.5, size=z16.shape).astype(np.float32)
    z = np.clip(z, 0.0, np.asarray(qmax, dtype=np.float32))   # qmax: a number, or one per row
    return s.astype(np.float16), z.astype(np.float16)


# ----------------------------------------------------------------------------
# The five workloads.  Each linear is (name, K, N, bits); M lists the batch
# sizes it is run at.  ``rht`` says whether activations are rotated.
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Linear:
    name: str
    k: int
    n: int
    bits: int            # 3, 4, 6, 8; 0 = mixed 6/8 in 64-row blocks
    rht: bool = True
    out_f32: bool = False


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    title: str
    linears: tuple
    ms: tuple
    extra: dict = field(default_factory=dict)


def _block(bits: int) -> tuple:
    return tuple(Linear(n, k, nn, bits) for (n, k, nn) in PROJECTIONS)


WORKLOADS = {
    "single_int4": Workload(
        0, "single_int4", "single linear 1024->512, int4 g128, RHT, M=1",
        (Linear("linear", 1024, 512, 4),), (1,)),
    "block_int4": Workload(
        1, "block_int4", "4B-class decoder block, 7 projections, int4 g128, RHT",
        _block(4), (1, 4)),
    "block_int3": Workload(
        2, "block_int3", "4B-class decoder block, 7 projections, int3 g128, RHT",
        _block(3), (1, 4, 16)),
    "block_int6_head_int8": Workload(
        3, "block_int6_head_int8",
        "7 projections int6 g128 with RHT, plus 151936x2560 int8 g128 head without RHT (fp32 logits)",
        _block(6) + (Linear(HEAD[0], HEAD[1], HEAD[2], 8, rht=False, out_f32=True),), (1,)),
    "prefill_and_mixed": Workload(
        4, "prefill_and_mixed",
        "A: 7 projections int4 g128 with RHT at M=512; B: down_proj 9728->2560 mixed 6/8-bit 64-row blocks at M=1",
        _block(4) + (Linear("down_proj_mixed", 9728, 2560, 0),), (512, 1)),
}


def linear_inputs(seed: int, wid: int, index: int, lin: Linear, m: int):
    """Weight, activations, sign bits and (mixed width only) selectors for one linear.

    Tensor ids: 4*index + {0: weight, 1: signs, 2: activations, 3: selectors}.
    Activations get ``m`` folded into their stream so each batch size draws
    its own rows.
    """
    w = weight(lin.k, lin.n, rng_for(seed, wid, 4 * index + 0))
    signs = sign_bits(lin.k, rng_for(seed, wid, 4 * index + 1)) if lin.rht else None
    x = activations(m, lin.k, np.random.default_rng(
        np.random.SeedSequence([seed, wid, 4 * index + 2, m])))
    sel = block_selector(lin.n, rng_for(seed, wid, 4 * index + 3)) if lin.bits == 0 else None
    return w, x, signs, sel


def weight_rows(seed: int, wid: int, index: int, lin: Linear, rows: np.ndarray) -> np.ndarray:
    """The given output rows of ``linear_inputs(...)[0]`` without keeping all of it.

    Draws the full matrix in row chunks from the same stream, so it returns
    exactly the same values while holding at most one chunk at a time.
    Used where only a sample of a very large matrix is needed.
    """
    # standard_normal fills row-major, so drawing in row chunks from one
    # generator reproduces the single full draw exactly.
    rng = rng_for(seed, wid, 4 * index + 0)
    rows = np.asarray(rows)
    out = np.empty((len(rows), lin.k), dtype=np.float32)
    chunk = max(1, (1 << 24) // lin.k)
    for r0 in range(0, lin.n, chunk):
        r1 = min(lin.n, r0 + chunk)
        block = rng.standard_normal((r1 - r0, lin.k), dtype=np.float32)
        hit = np.nonzero((rows >= r0) & (rows < r1))[0]
        if len(hit):
            out[hit] = block[rows[hit] - r0]
    out *= np.float32(0.02)
    n_out = int(round(0.01 * lin.k))
    if n_out:
        idx = rng.choice(lin.k, n_out, replace=False)
        out[:, idx] *= np.float32(20.0)
    return out
