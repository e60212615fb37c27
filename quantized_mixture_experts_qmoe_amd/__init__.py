"""Python binding of libqmoe, the gfx950 quantized MoE layer.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the layer runs in the library's HIP kernels. There
is no CPU fallback: if ``libqmoe.so`` is missing or fails to load, every entry
point raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")

QMOE_F32, QMOE_BF16, QMOE_F16 = 0, 1, 2
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
          3: "workspace missing or too small", 4: "HIP runtime error", 5: "out of host memory"}

EXPORTS = ("qmoe_create", "qmoe_workspace_size", "qmoe_forward", "qmoe_destroy",
           "qmoe_status_string", "qmoe_route", "qmoe_dequant", "qmoe_workspace_routing",
           "qmoe_set_stage_hook", "qmoe_decode_errors", "qmoe_forward_noalloc")
NOALLOC_WORKSPACE_BYTES = 32 << 20   # QMOE_NOALLOC_WORKSPACE_BYTES (include/qmoe.h)

STAGE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p)


class QMoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("top_k", ctypes.c_int32),
                ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
                ("num_experts", ctypes.c_int64), ("bits", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("zero_point", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("normalize_routing", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("max_tokens", ctypes.c_int64)]


QMOE_FLAG_FC1_INTERLEAVED = 1   # qmoe_config.flags bit (include/qmoe.h)


class Weights(ctypes.Structure):
    _fields_ = [("fc1_codes", ctypes.c_void_p), ("fc1_scales", ctypes.c_void_p),
                ("fc2_codes", ctypes.c_void_p), ("fc2_scales", ctypes.c_void_p),
                ("fc1_bias", ctypes.c_void_p), ("fc2_bias", ctypes.c_void_p),
                ("fc1_zero_points", ctypes.c_void_p), ("fc2_zero_points", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqmoe.so (built in-tree by ``_build.build``); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m quantized_mixture_experts_qmoe_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.qmoe_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), ctypes.c_int,
                                  ctypes.POINTER(P)]
        L.qmoe_workspace_size.argtypes = [P, i64, ctypes.POINTER(sz)]
        L.qmoe_forward.argtypes = [P, P, P, P, i64, P, sz, P]
        L.qmoe_destroy.argtypes = [P]
        L.qmoe_status_string.argtypes = [i32]
        L.qmoe_status_string.restype = ctypes.c_char_p
        L.qmoe_route.argtypes = [P, P, i64, P, P, P, P, P, P, sz, P]
        L.qmoe_dequant.argtypes = [P, ctypes.c_int, i64, P, P, P]
        L.qmoe_workspace_routing.argtypes = [P, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.qmoe_set_stage_hook.argtypes = [P, STAGE_FN, P]
        L.qmoe_decode_errors.argtypes = [P, P, ctypes.POINTER(ctypes.c_uint32)]
        L.qmoe_forward_noalloc.argtypes = [P, P, P, P, i64, P]
        for name in ("qmoe_create", "qmoe_workspace_size", "qmoe_forward", "qmoe_destroy",
                     "qmoe_route", "qmoe_dequant", "qmoe_workspace_routing", "qmoe_set_stage_hook",
                     "qmoe_decode_errors", "qmoe_forward_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(st: int, what: str):
    if st != 0:
        raise QMoEError(st, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream: Optional[torch.cuda.Stream] = None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


_ACT = {torch.bfloat16: QMOE_BF16, torch.float32: QMOE_F32, torch.float16: QMOE_F16}


@dataclass
class LayerConfig:
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    bits: int
    block_size: int
    zero_point: int = -1
    act_dtype: torch.dtype = torch.bfloat16
    max_tokens: int = 8192
    normalize_routing: bool = True   # False: weights over all experts, not renormalized over the k
    fc1_interleaved: bool = False    # FC1 rows 2n / 2n+1 = gate n / up n (else gate block, up block)


def check_weight_shapes(cfg: LayerConfig, fc1_codes, fc1_scales, fc2_codes, fc2_scales):
    """Raise ValueError unless the four weight tensors have the layout the
    library reads: codes uint8 [E, N, K*bits/8] and scales fp16 [E, N, K/bs],
    N x K = 2I x H for FC1 and H x I for FC2. The library cannot check sizes
    behind raw pointers, and a tensor that is too small would be read out of
    bounds on the GPU."""
    E, H, I, b, bs = cfg.num_experts, cfg.hidden, cfg.inter, cfg.bits, cfg.block_size
    if b not in (2, 3, 4) or bs not in (32, 64, 128) or H <= 0 or I <= 0 or H % bs or I % bs:
        raise ValueError("bits must be 2, 3 or 4 and block_size 32, 64 or 128, dividing hidden "
                         "and inter")
    want = (("fc1_codes", fc1_codes, (E, 2 * I, H * b // 8)),
            ("fc1_scales", fc1_scales, (E, 2 * I, H // bs)),
            ("fc2_codes", fc2_codes, (E, H, I * b // 8)),
            ("fc2_scales", fc2_scales, (E, H, I // bs)))
    for name, t, shape in want:
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be shaped {shape}, got {tuple(t.shape)}")


class QMoELayer:
    """One quantized MoE layer resident on a GPU.

    Weight tensors (on the GPU, contiguous, owned by the caller and kept alive
    by this object): fc1_codes uint8 [E, 2I, H*bits/8], fc1_scales fp16
    [E, 2I, H/bs], fc2_codes uint8 [E, H, I*bits/8], fc2_scales fp16 [E, H, I/bs];
    optional fc1_bias [E, 2I] and fc2_bias [E, H] in the activation dtype, and
    optional uint8 zero-point tensors shaped like the scales.
    """

    def __init__(self, cfg: LayerConfig, fc1_codes: torch.Tensor, fc1_scales: torch.Tensor,
                 fc2_codes: torch.Tensor, fc2_scales: torch.Tensor,
                 fc1_bias: Optional[torch.Tensor] = None, fc2_bias: Optional[torch.Tensor] = None,
                 fc1_zero_points: Optional[torch.Tensor] = None,
                 fc2_zero_points: Optional[torch.Tensor] = None):
        check_weight_shapes(cfg, fc1_codes, fc1_scales, fc2_codes, fc2_scales)
        for t in (fc1_codes, fc1_scales, fc2_codes, fc2_scales):
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("weights must be contiguous GPU tensors")
        for t, shape in ((fc1_bias, (cfg.num_experts, 2 * cfg.inter)),
                         (fc2_bias, (cfg.num_experts, cfg.hidden))):
            if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != cfg.act_dtype
                                  or tuple(t.shape) != shape):
                raise ValueError(f"biases must be contiguous GPU tensors of the activation dtype, "
                                 f"shaped {shape}")
        for t, sc in ((fc1_zero_points, fc1_scales), (fc2_zero_points, fc2_scales)):
            if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != torch.uint8
                                  or t.shape != sc.shape):
                raise ValueError("zero points must be contiguous uint8 GPU tensors shaped like "
                                 "the scales")
        if fc1_codes.dtype != torch.uint8 or fc2_codes.dtype != torch.uint8:
            raise ValueError("codes must be uint8")
        if fc1_scales.dtype != torch.float16 or fc2_scales.dtype != torch.float16:
            raise ValueError("scales must be float16")
        if cfg.act_dtype not in _ACT:
            raise ValueError("act_dtype must be torch.bfloat16, torch.float16 or torch.float32")
        self.cfg = cfg
        self.device = fc1_codes.device
        self._keep = (fc1_codes, fc1_scales, fc2_codes, fc2_scales, fc1_bias, fc2_bias,
                      fc1_zero_points, fc2_zero_points)
        c = Config(ctypes.sizeof(Config), cfg.top_k, cfg.hidden, cfg.inter, cfg.num_experts,
                   cfg.bits, cfg.block_size, cfg.zero_point, _ACT[cfg.act_dtype],
                   1 if cfg.normalize_routing else 0,
                   QMOE_FLAG_FC1_INTERLEAVED if cfg.fc1_interleaved else 0, cfg.max_tokens)
        w = Weights(fc1_codes.data_ptr(), fc1_scales.data_ptr(), fc2_codes.data_ptr(),
                    fc2_scales.data_ptr(), None if fc1_bias is None else fc1_bias.data_ptr(),
                    None if fc2_bias is None else fc2_bias.data_ptr(),
                    None if fc1_zero_points is None else fc1_zero_points.data_ptr(),
                    None if fc2_zero_points is None else fc2_zero_points.data_ptr())
        h = ctypes.c_void_p()
        _check(lib().qmoe_create(ctypes.byref(c), ctypes.byref(w), self.device.index or 0,
                                 ctypes.byref(h)), "qmoe_create")
        self._h = h
        self._ws: Optional[torch.Tensor] = None

    def close(self):
        if getattr(self, "_h", None):
            lib().qmoe_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, num_tokens: int) -> int:
        n = ctypes.c_size_t()
        _check(lib().qmoe_workspace_size(self._h, num_tokens, ctypes.byref(n)), "qmoe_workspace_size")
        return n.value

    def workspace(self, num_tokens: int) -> torch.Tensor:
        need = self.workspace_size(num_tokens)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def _check_tokens(self, x: torch.Tensor, logits: torch.Tensor):
        c = self.cfg
        if x.dtype != c.act_dtype or logits.dtype != c.act_dtype:
            raise ValueError("x and logits must have the layer's activation dtype")
        if x.dim() != 2 or x.shape[1] != c.hidden or logits.shape != (x.shape[0], c.num_experts):
            raise ValueError("expected x [T, hidden] and logits [T, num_experts]")
        if x.device != self.device or logits.device != self.device:
            raise ValueError("x and logits must be on the layer's device")
        if not x.is_contiguous() or not logits.is_contiguous():
            raise ValueError("x and logits must be contiguous")

    def forward(self, x: torch.Tensor, logits: torch.Tensor, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        """x [T, hidden] or [batch, seq, hidden]; logits [T, num_experts], or for
        3-D x [batch, seq, num_experts] or [batch * seq, num_experts]. A 3-D
        input is the same packed token-major rows (batch * seq tokens, viewed
        without a copy); the output has x's shape."""
        shape = x.shape
        if x.dim() == 3:
            if not x.is_contiguous() or not logits.is_contiguous():
                raise ValueError("x and logits must be contiguous")
            if logits.dim() == 3 and logits.shape[:2] != x.shape[:2]:
                raise ValueError("3-D logits must match x's [batch, seq]")
            x = x.view(-1, x.shape[-1])
            logits = logits.view(-1, logits.shape[-1])
        self._check_tokens(x, logits)
        T = x.shape[0]
        if out is None:
            out = torch.empty(shape, dtype=x.dtype, device=x.device)
        elif out.shape != shape or out.dtype != x.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor shaped and typed like x")
        ws = workspace if workspace is not None else self.workspace(T)
        _check(lib().qmoe_forward(self._h, _ptr(x), _ptr(logits), _ptr(out), T, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream()), "qmoe_forward")
        return out

    __call__ = forward

    def routing_from_workspace(self, num_tokens: int, workspace: torch.Tensor):
        """(topk_id [T, k] int32, topk_w [T, k] fp32) left in `workspace` by forward()."""
        a, b = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().qmoe_workspace_routing(self._h, num_tokens, ctypes.byref(a), ctypes.byref(b)),
               "qmoe_workspace_routing")
        R = num_tokens * self.cfg.top_k
        ids = workspace[a.value:a.value + 4 * R].view(torch.int32).view(num_tokens, self.cfg.top_k)
        w = workspace[b.value:b.value + 4 * R].view(torch.float32).view(num_tokens, self.cfg.top_k)
        return ids, w

    def decode_errors(self, stream: Optional[torch.cuda.Stream] = None) -> int:
        """Error bits of the fused decode's bounded waits since the last query
        (bit 0: an FC1 result wait ran out, bit 1: an FC2 result wait); waits
        for the stream, then clears them. 0 means every wait was met."""
        bits = ctypes.c_uint32()
        _check(lib().qmoe_decode_errors(self._h, _stream(stream), ctypes.byref(bits)),
               "qmoe_decode_errors")
        return bits.value

    def set_stage_hook(self, fn):
        """fn(stage: int, name: str) runs on the host after each kernel launch of
        forward(); None removes it."""
        if fn is None:
            self._hook = STAGE_FN()
        else:
            self._hook = STAGE_FN(lambda _u, stage, name: fn(stage, name.decode()))
        _check(lib().qmoe_set_stage_hook(self._h, self._hook, None), "qmoe_set_stage_hook")

    def route(self, logits: torch.Tensor):
        """Routing stage only: (topk_id, topk_w, expert_offsets, sorted_routes, inv_pos)."""
        c = self.cfg
        T = logits.shape[0]
        if logits.dtype != c.act_dtype or logits.shape != (T, c.num_experts) or not logits.is_contiguous():
            raise ValueError("logits must be contiguous [T, num_experts] of the activation dtype")
        R = T * c.top_k
        dev = self.device
        ids = torch.empty((T, c.top_k), dtype=torch.int32, device=dev)
        w = torch.empty((T, c.top_k), dtype=torch.float32, device=dev)
        offs = torch.empty(c.num_experts + 1, dtype=torch.int32, device=dev)
        srt = torch.empty(R, dtype=torch.int32, device=dev)
        inv = torch.empty(R, dtype=torch.int32, device=dev)
        ws = self.workspace(T)
        _check(lib().qmoe_route(self._h, _ptr(logits), T, _ptr(ids), _ptr(w), _ptr(offs), _ptr(srt),
                                _ptr(inv), _ptr(ws), ws.numel(), _stream()), "qmoe_route")
        return ids, w, offs, srt, inv

    def dequant(self, fc: int, expert: int):
        """(fp32 [N, K] as the decode path reads it, fp16 [N, K] as the prefill path stages it)."""
        c = self.cfg
        N, K = (2 * c.inter, c.hidden) if fc == 1 else (c.hidden, c.inter)
        f = torch.empty((N, K), dtype=torch.float32, device=self.device)
        b = torch.empty((N, K), dtype=torch.int16, device=self.device)
        _check(lib().qmoe_dequant(self._h, fc, expert, _ptr(f), _ptr(b), _stream()), "qmoe_dequant")
        return f, b.view(torch.float16)
