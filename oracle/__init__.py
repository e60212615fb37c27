"""CPU oracle for the quantized MoE layer: ctypes binding to ``qmoe_oracle.c``.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package. The GPU library (``quantized_mixture_experts_qmoe_amd``) never
imports it, and the two share no code.

Every function takes host numpy arrays. Activations and logits are widened to
float64 before the call; that widening is exact for bf16 and fp32 inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmoe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_qmoe.so")

# Rounding points of the fp16 matrix-core datapath (qmoe_oracle.c describes
# each): activations, dequantized weights, SwiGLU output.
EMU_X_F16 = 1
EMU_W_F16 = 2
EMU_H_F16 = 4
EMU_F16_DATAPATH = EMU_X_F16 | EMU_W_F16 | EMU_H_F16
EMU_W_BF16 = 8      # the earlier bf16 datapath: weights and h rounded to bf16
EMU_H_BF16 = 16


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
                ("num_experts", ctypes.c_int64), ("top_k", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("zero_point", ctypes.c_int32), ("emulate", ctypes.c_int32),
                ("normalize", ctypes.c_int32), ("fc1_interleaved", ctypes.c_int32),
                ("pad", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.oracle_dequant.argtypes = [P, P, i64, i64, i32, i32, i32, P]
        L.oracle_route.argtypes = [P, i64, i64, i32, i32, P, P]
        L.oracle_permute.argtypes = [P, i64, i64, P, P, P, P]
        L.oracle_forward.argtypes = [ctypes.POINTER(_Layer), P, P, P, P, P, P, i64, P, i32]
        L.oracle_forward_ext.argtypes = [ctypes.POINTER(_Layer), P, P, P, P, P, P, P, P, P, P, i64, P,
                                         i32]
        L.oracle_dequant_zp.argtypes = [P, P, P, i64, i64, i32, i32, i32, P]
        L.oracle_dequant_f16.argtypes = [P, P, P, i64, i64, i32, i32, i32, P]
        L.oracle_double_to_half_n.argtypes = [P, i64, P]
        L.oracle_double_to_half_n.restype = None
        L.oracle_emulate_x_rows.argtypes = [P, i64, i64, P]
        L.oracle_emulate_x_rows.restype = None
        L.oracle_emulate_h_rows.argtypes = [P, i64, i64]
        L.oracle_emulate_h_rows.restype = None
        L.oracle_round_output.argtypes = [P, i64, P, P]
        L.oracle_round_output.restype = None
        L.oracle_half_to_double_n.argtypes = [P, i64, P]
        L.oracle_half_to_double_n.restype = None
        L.oracle_f32_to_bf16_n.argtypes = [P, i64, P]
        L.oracle_f32_to_bf16_n.restype = None
        for f in (L.oracle_dequant, L.oracle_route, L.oracle_permute, L.oracle_forward,
                  L.oracle_forward_ext, L.oracle_dequant_zp, L.oracle_dequant_f16):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    """Pointer to a C-contiguous array (None for an absent optional input)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(st: int, what: str):
    if st != 0:
        raise ValueError(f"oracle {what} failed with status {st}")


def as_f64(t) -> np.ndarray:
    """Exact widening of a bf16/fp32 torch tensor or numpy array to float64."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return np.ascontiguousarray(t.detach().cpu().to(torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(t, dtype=np.float64))


def half_to_double(h_bits: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h_bits, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    lib().oracle_half_to_double_n(_p(h), h.size, _p(out))
    return out


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_n(_p(f), f.size, _p(out))
    return out


def double_to_half_bits(v: np.ndarray) -> np.ndarray:
    """Nearest fp16 (ties to even, gradual underflow) of float64 values, as bits."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_double_to_half_n(_p(v), v.size, _p(out))
    return out


def emulate_x_rows(x: np.ndarray) -> np.ndarray:
    """Rows of activations as the fp16 datapath's FC1 reads them (EMU_X_F16)."""
    x = np.array(x, dtype=np.float64, order="C", copy=True)
    tmp = np.empty(x.shape[-1], dtype=np.float64)
    lib().oracle_emulate_x_rows(_p(x), x.size // x.shape[-1], x.shape[-1], _p(tmp))
    return x


def emulate_h_rows(h: np.ndarray) -> np.ndarray:
    """Rows of SwiGLU outputs as the fp16 datapath's FC2 reads them (EMU_H_F16)."""
    h = np.array(h, dtype=np.float64, order="C", copy=True)
    lib().oracle_emulate_h_rows(_p(h), h.size // h.shape[-1], h.shape[-1])
    return h


def dequant_f16(codes: np.ndarray, scales: np.ndarray, bits: int, block_size: int,
                zero_point: int, K: int, zero_points: Optional[np.ndarray] = None) -> np.ndarray:
    """fp16((q - zp) * s) bit patterns (uint16 [N, K]): the weight operand of
    the fp16 datapath."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(scales).view(np.uint16)
    zps = None if zero_points is None else np.ascontiguousarray(zero_points, dtype=np.uint8)
    N = codes.shape[0]
    assert zps is None or zps.shape == sc.shape
    out = np.empty((N, K), dtype=np.uint16)
    _check(lib().oracle_dequant_f16(_p(codes), _p(sc), _p(zps), N, K, bits, block_size,
                                    zero_point, _p(out)), "dequant_f16")
    return out


def dequant(codes: np.ndarray, scales: np.ndarray, bits: int, block_size: int,
            zero_point: int, K: int, zero_points: Optional[np.ndarray] = None) -> np.ndarray:
    """(q - zp) * s for one [N, K] matrix of packed codes -> float64 [N, K];
    zero_points (uint8 [N, K/bs]) replaces the scalar zero point when given."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(scales).view(np.uint16)
    zps = None if zero_points is None else np.ascontiguousarray(zero_points, dtype=np.uint8)
    N = codes.shape[0]
    assert zps is None or zps.shape == sc.shape
    out = np.empty((N, K), dtype=np.float64)
    _check(lib().oracle_dequant_zp(_p(codes), _p(sc), _p(zps), N, K, bits, block_size, zero_point,
                                   _p(out)), "dequant")
    return out


def route(logits, k: int, normalize: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k ids (int32 [T, k]) and routing weights (float64 [T, k]): the
    softmax over the selected logits, or with normalize=False each selected
    expert's softmax probability over all E logits."""
    l64 = as_f64(logits)
    T, E = l64.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    _check(lib().oracle_route(_p(l64), T, E, k, int(bool(normalize)), _p(ids), _p(w)), "route")
    return ids, w


def permute(topk_id: np.ndarray, num_experts: int):
    """counts [E], expert_offsets [E+1], sorted_routes [R], inv_pos [R] (int32)."""
    ids = np.ascontiguousarray(topk_id, dtype=np.int32).reshape(-1)
    R = ids.size
    counts = np.empty(num_experts, dtype=np.int32)
    offsets = np.empty(num_experts + 1, dtype=np.int32)
    sorted_routes = np.empty(R, dtype=np.int32)
    inv_pos = np.empty(R, dtype=np.int32)
    _check(lib().oracle_permute(_p(ids), R, num_experts, _p(counts), _p(offsets),
                                _p(sorted_routes), _p(inv_pos)), "permute")
    return counts, offsets, sorted_routes, inv_pos


@dataclass
class Layer:
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    bits: int
    block_size: int
    zero_point: int
    normalize: bool = True   # routing weights over the selected k (else over all experts)
    fc1_interleaved: bool = False   # FC1 rows 2n / 2n+1 = gate n / up n (else two blocks)

    @classmethod
    def from_spec(cls, spec, normalize: bool = True, fc1_interleaved: bool = False) -> "Layer":
        return cls(spec.hidden, spec.inter, spec.num_experts, spec.top_k, spec.bits,
                   spec.block_size, spec.zero_point, normalize, fc1_interleaved)


def forward(layer: Layer, x, logits, weights, *, nthreads: Optional[int] = None,
            emulate: int = 0, fc1_bias=None, fc2_bias=None, fc1_zero_points=None,
            fc2_zero_points=None) -> np.ndarray:
    """Whole layer in double precision; returns the float64 accumulator [T, H].
    fc1_bias [E, 2I] and fc2_bias [E, H] (optional, any float dtype, read as
    exact values) are added to FC1 rows before SwiGLU and to y before the
    routing-weighted sum. fc1_zero_points / fc2_zero_points (uint8, shaped
    like the scales) replace the scalar zero point per row and quant block.
    emulate: a bitmask of EMU_* rounding points (0: the plain definition)."""
    x64 = as_f64(x)
    l64 = as_f64(logits)
    T = x64.shape[0]
    assert x64.shape == (T, layer.hidden) and l64.shape == (T, layer.num_experts)
    c1 = np.ascontiguousarray(weights.fc1_codes, dtype=np.uint8)
    s1 = np.ascontiguousarray(weights.fc1_scales).view(np.uint16)
    c2 = np.ascontiguousarray(weights.fc2_codes, dtype=np.uint8)
    s2 = np.ascontiguousarray(weights.fc2_scales).view(np.uint16)
    E, H, I = layer.num_experts, layer.hidden, layer.inter
    assert c1.shape == (E, 2 * I, H * layer.bits // 8) and s1.shape == (E, 2 * I, H // layer.block_size)
    assert c2.shape == (E, H, I * layer.bits // 8) and s2.shape == (E, H, I // layer.block_size)
    out = np.empty((T, H), dtype=np.float64)
    L = _Layer(H, I, E, layer.top_k, layer.bits, layer.block_size, layer.zero_point, emulate,
               int(bool(layer.normalize)), int(bool(layer.fc1_interleaved)), 0)
    if nthreads is None:
        nthreads = default_threads()
    b1 = None if fc1_bias is None else as_f64(fc1_bias)
    b2 = None if fc2_bias is None else as_f64(fc2_bias)
    assert b1 is None or b1.shape == (E, 2 * I)
    assert b2 is None or b2.shape == (E, H)
    z1 = None if fc1_zero_points is None else np.ascontiguousarray(fc1_zero_points, dtype=np.uint8)
    z2 = None if fc2_zero_points is None else np.ascontiguousarray(fc2_zero_points, dtype=np.uint8)
    assert z1 is None or z1.shape == s1.shape
    assert z2 is None or z2.shape == s2.shape
    _check(lib().oracle_forward_ext(ctypes.byref(L), _p(x64), _p(l64), _p(c1), _p(s1), _p(c2),
                                    _p(s2), _p(b1), _p(b2), _p(z1), _p(z2), T, _p(out), nthreads),
           "forward")
    return out


def round_output(acc: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """fp32 result (one rounding of the double accumulator) and its bf16 bits."""
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    f = np.empty(acc.shape, dtype=np.float32)
    b = np.empty(acc.shape, dtype=np.uint16)
    lib().oracle_round_output(_p(acc), acc.size, _p(f), _p(b))
    return f, b


_THREADS = None


def default_threads() -> int:
    """Cores available to this process, resolved once."""
    global _THREADS
    if _THREADS is None:
        try:
            _THREADS = max(1, len(os.sched_getaffinity(0)))
        except AttributeError:  # pragma: no cover
            _THREADS = os.cpu_count() or 1
    return _THREADS
