"""Helpers shared by the GPU parity tests (host-side only)."""
import os
import sys

import numpy as np
import torch

import oracle
import qmoe_inputs as qi
import quantized_mixture_experts_qmoe_amd as q

DEV = torch.device("cuda:0")


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def layer_for(wl: qi.Workload, max_tokens: int = 8192, normalize: bool = True,
              fc1_interleaved: bool = False, fc1_bias=None, fc2_bias=None,
              fc1_zero_points=None, fc2_zero_points=None) -> q.QMoELayer:
    s = wl.spec
    w = wl.weights
    cfg = q.LayerConfig(s.hidden, s.inter, s.num_experts, s.top_k, s.bits, s.block_size,
                        s.zero_point, qi.TORCH_DTYPE[s.act_dtype],
                        max_tokens, normalize, fc1_interleaved)
    return q.QMoELayer(cfg, torch.from_numpy(w.fc1_codes).to(DEV),
                       torch.from_numpy(w.fc1_scales).to(DEV), torch.from_numpy(w.fc2_codes).to(DEV),
                       torch.from_numpy(w.fc2_scales).to(DEV),
                       None if fc1_bias is None else fc1_bias.to(DEV),
                       None if fc2_bias is None else fc2_bias.to(DEV),
                       None if fc1_zero_points is None else torch.from_numpy(fc1_zero_points).to(DEV),
                       None if fc2_zero_points is None else torch.from_numpy(fc2_zero_points).to(DEV))


def run(layer: q.QMoELayer, x: torch.Tensor, logits: torch.Tensor):
    ws = layer.workspace(x.shape[0])
    out = layer(x.to(DEV), logits.to(DEV), workspace=ws)
    torch.cuda.synchronize()
    return out, ws


def oracle_acc(wl: qi.Workload, rows=None) -> np.ndarray:
    x, l = wl.tokens.x, wl.tokens.logits
    if rows is not None:
        idx = torch.as_tensor(rows, dtype=torch.long)
        x, l = x[idx], l[idx]
    return oracle.forward(oracle.Layer.from_spec(wl.spec), x, l, wl.weights)


def sample_rows(T: int, n: int, seed: int) -> np.ndarray:
    """n distinct token indices including the first and the last token."""
    rng = np.random.default_rng(seed)
    n = min(n, T)
    rows = set([0, T - 1])
    rows.update(rng.choice(T, size=n, replace=False).tolist())
    return np.array(sorted(rows))[: max(n, 2)] if T > 1 else np.array([0])


def fp32_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ai = a.astype(np.float32).view(np.int32).astype(np.int64)
    bi = b.astype(np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)
