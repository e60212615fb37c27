"""Independent numpy (float64) formulations used to pin the C oracle.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

These are deliberately written differently from ``qmoe_oracle.c`` so that one
mistake cannot hide in both:

- codes are read as one little-endian bit stream (``np.unpackbits`` with
  ``bitorder='little'``) cut into consecutive ``bits``-wide fields, instead of
  per-format shifts and masks. For INT4 (low nibble first), INT2 (low bits
  first) and INT3 (code i at bits [3i, 3i+3) of the little-endian 24-bit
  word) that stream reading is the same packing;
- scales are expanded with ``np.repeat`` over the block and multiplied in bulk;
- top-k is a full stable sort by (-logit, expert index) (``np.lexsort``);
- the layer is computed densely: every expert runs on every token through
  BLAS matmuls, and a [T, E] gate matrix that is zero off the top-k selects
  and weights the results (a masked mixture), instead of per-route loops;
- the fp16 rounding points of the emulated datapath use numpy's own float64
  -> float16 conversion and whole-array exponent arithmetic (``np.frexp``,
  ``np.ldexp``) over reshaped chunks, instead of the C oracle's hand-written
  rounding and per-element loops.
"""
from __future__ import annotations

import numpy as np


def unpack_codes(codes: np.ndarray, bits: int, K: int) -> np.ndarray:
    """uint8 [..., K*bits/8] -> int64 [..., K] via a little-endian bit stream."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    lead = codes.shape[:-1]
    stream = np.unpackbits(codes, axis=-1, bitorder="little")          # [..., 8*nbytes]
    fields = stream.reshape(*lead, K, bits).astype(np.int64)
    weights = (1 << np.arange(bits, dtype=np.int64))
    return (fields * weights).sum(axis=-1)


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """int [..., K] codes in [0, 2^bits) -> uint8 [..., K*bits/8] (little-endian bit stream)."""
    q = np.asarray(q, dtype=np.int64)
    assert q.min(initial=0) >= 0 and q.max(initial=0) < (1 << bits)
    lead, K = q.shape[:-1], q.shape[-1]
    assert (K * bits) % 8 == 0
    bitsarr = ((q[..., None] >> np.arange(bits)) & 1).astype(np.uint8)   # [..., K, bits]
    stream = bitsarr.reshape(*lead, K * bits)
    return np.packbits(stream, axis=-1, bitorder="little")


def dequant_dense(codes: np.ndarray, scales: np.ndarray, bits: int, block_size: int,
                  zero_point, K: int) -> np.ndarray:
    """zero_point: a scalar code, or an array of codes shaped like scales."""
    q = unpack_codes(codes, bits, K)
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), block_size, axis=-1)
    z = zero_point
    if isinstance(z, np.ndarray):
        z = np.repeat(z.astype(np.int64), block_size, axis=-1)
    return (q.astype(np.int64) - z).astype(np.float64) * s


def topk_brute(logits64: np.ndarray, k: int) -> np.ndarray:
    """Stable full sort of every token's experts by (-logit, index); first k ids."""
    T, E = logits64.shape
    idx = np.arange(E)
    out = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((idx, -logits64[t]))     # primary: -logit, secondary: index
        out[t] = order[:k]
    return out


def softmax_selected(logits64: np.ndarray, ids: np.ndarray) -> np.ndarray:
    sel = np.take_along_axis(logits64, ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def f16(v: np.ndarray) -> np.ndarray:
    """Nearest float16 value (numpy's conversion), back in float64."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float64)


def _range_exponent(M: np.ndarray, lo: float) -> np.ndarray:
    """0 where M (finite, >= 0) is 0 or lies in [lo, 2^15], else the e with
    M * 2^-e in [2^14, 2^15), clamped to [-120, 120]."""
    e = np.clip(np.frexp(np.where(M > 0, M, 1.0))[1].astype(np.int64) - 15, -120, 120)
    return np.where((M == 0) | ((M >= lo) & (M <= 32768.0)), 0, e)


def f16_rows_scaled(x: np.ndarray) -> np.ndarray:
    """Each row rounded to fp16 after an exact scaling by its range exponent
    (lower bound 2^-3; rows with a non-finite value: no scaling)."""
    finite = np.isfinite(x).all(axis=-1, keepdims=True)
    M = np.where(finite, np.abs(np.where(np.isfinite(x), x, 0.0)).max(axis=-1, keepdims=True), 0.0)
    e = _range_exponent(M, 2.0 ** -3)
    return np.ldexp(f16(np.ldexp(x, -e)), e)


def f16_chunks_scaled(h: np.ndarray, chunk: int = 32, *, plant_no_chunk_exponent: bool = False,
                      plant_no_common_exponent: bool = False) -> np.ndarray:
    """h [..., I] as FC2 of the fp16 datapath reads it: per chunk of 32 values,
    the range exponent of the chunk (lower bound 2^-14; none for a chunk
    with a non-finite value); each chunk stored as fp16 at its exponent, then brought to the
    row's largest chunk exponent E with a second fp16 rounding. The plant_*
    switches drop one step (for the pin tests)."""
    lead, I = h.shape[:-1], h.shape[-1]
    c = h.reshape(*lead, I // chunk, chunk)
    finite = np.isfinite(c).all(axis=-1, keepdims=True)
    M = np.where(finite, np.abs(np.where(np.isfinite(c), c, 0.0)).max(axis=-1, keepdims=True), 0.0)
    e = _range_exponent(M, 2.0 ** -14)
    if plant_no_chunk_exponent:
        e = np.zeros_like(e)
    stored = f16(np.ldexp(c, -e))
    E = e.max(axis=-2, keepdims=True)
    if plant_no_common_exponent:
        return np.ldexp(stored, e).reshape(h.shape)
    return np.ldexp(f16(np.ldexp(stored, e - E)), E).reshape(h.shape)


def silu(v: np.ndarray) -> np.ndarray:
    return v * (0.5 * (1.0 + np.tanh(0.5 * v)))      # sigmoid via tanh identity


def dense_masked_forward(x64: np.ndarray, logits64: np.ndarray, weights, spec,
                         *, swap_gate_up: bool = False, zp_delta: int = 0,
                         softmax_all: bool = False, fc1_bias=None, fc2_bias=None,
                         bias_after_silu: bool = False, fc1_zero_points=None,
                         fc2_zero_points=None, emu_x: bool = False, emu_w: bool = False,
                         emu_h: bool = False, plant_h_unrounded: bool = False,
                         plant_h_no_chunk_exponent: bool = False,
                         plant_h_no_common_exponent: bool = False,
                         plant_x_unscaled: bool = False) -> np.ndarray:
    """Masked-mixture formulation of the layer in float64.

    emu_x / emu_w / emu_h apply the fp16 datapath's rounding points to the
    activations, the dequantized weights and the SwiGLU output.
    The other keyword switches plant deliberate mistakes; tests use them to
    show that the comparison against the oracle would notice each one.
    """
    T = x64.shape[0]
    E, H, I, k = spec.num_experts, spec.hidden, spec.inter, spec.top_k
    if emu_x:
        x64 = f16(x64) if plant_x_unscaled else f16_rows_scaled(x64)
    ids = topk_brute(logits64, k)
    if softmax_all:
        z = np.exp(logits64 - logits64.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, ids, axis=1)
    else:
        w = softmax_selected(logits64, ids)
    gate = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(gate, ids, w, axis=1)
    out = np.zeros((T, H), dtype=np.float64)
    zp = spec.zero_point + zp_delta
    for e in range(E):
        if not gate[:, e].any():
            continue
        z1 = zp if fc1_zero_points is None else fc1_zero_points[e].astype(np.int64) + zp_delta
        z2 = zp if fc2_zero_points is None else fc2_zero_points[e].astype(np.int64) + zp_delta
        W1 = dequant_dense(weights.fc1_codes[e], weights.fc1_scales[e], spec.bits,
                           spec.block_size, z1, H)                   # [2I, H]
        W2 = dequant_dense(weights.fc2_codes[e], weights.fc2_scales[e], spec.bits,
                           spec.block_size, z2, I)                   # [H, I]
        if emu_w:
            W1, W2 = f16(W1), f16(W2)
        gu = x64 @ W1.T                                             # [T, 2I]
        if fc1_bias is not None and not bias_after_silu:
            gu = gu + fc1_bias[e][None, :]
        g, u = gu[:, :I], gu[:, I:]
        if swap_gate_up:
            g, u = u, g
        h = silu(g) * u
        if fc1_bias is not None and bias_after_silu:
            h = h + fc1_bias[e][None, :I]
        if emu_h and not plant_h_unrounded:
            h = f16_chunks_scaled(h, plant_no_chunk_exponent=plant_h_no_chunk_exponent,
                                  plant_no_common_exponent=plant_h_no_common_exponent)
        y = h @ W2.T
        if fc2_bias is not None:
            y = y + fc2_bias[e][None, :]
        out += gate[:, e:e + 1] * y
    return out
