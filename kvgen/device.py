"""Upload generated inputs into torch device tensors (plumbing only).

``upload`` copies an in-memory ``kvgen.Inputs``; ``generate_on_device``
produces a workload slab by slab straight into device tensors, so caches of
tens of gigabytes never exist whole in host memory.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import kvgen


@dataclass
class DeviceInputs:
    workload: "kvgen.Workload"
    q: torch.Tensor
    k: tuple            # (data, scale or None)
    v: Optional[tuple]  # None when V aliases K
    seq_lens: torch.Tensor


def _t(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def upload(inp: "kvgen.Inputs", device="cuda") -> DeviceInputs:
    w = inp.workload
    k = (_t(inp.k_data, device), _t(inp.k_scale, device))
    v = None if w.v_aliases_k else (_t(inp.v_data, device), _t(inp.v_scale, device))
    return DeviceInputs(w, _t(inp.q, device), k, v, _t(inp.seq_lens, device))


def _empty_kv(w, D, device):
    shape = (w.B, w.Hkv, w.S_max)
    if w.kv_dtype == "f32":
        return torch.empty(shape + (D,), dtype=torch.float32, device=device), None
    if w.kv_dtype == "bf16":
        return torch.empty(shape + (D,), dtype=torch.int16, device=device), None
    if w.kv_dtype == "fp8":
        return (torch.empty(shape + (D,), dtype=torch.uint8, device=device),
                torch.empty((w.B, w.Hkv), dtype=torch.float32, device=device))
    if w.kv_dtype == "mxfp4":
        return (torch.empty(shape + (D // 2,), dtype=torch.uint8, device=device),
                torch.empty(shape + (D // 32,), dtype=torch.uint8, device=device))
    raise ValueError(w.kv_dtype)


def generate_on_device(w: "kvgen.Workload", device="cuda", threads=None, progress=None) -> DeviceInputs:
    """Generate w slab by slab into device tensors (host memory: one slab)."""
    q = _t(kvgen.gen_q(w, threads), device)
    seq = _t(kvgen.gen_seq_lens(w), device)
    out = {}
    for which in ("k",) if w.v_aliases_k else ("k", "v"):
        D = w.Dqk if which == "k" else w.Dv
        data, scale = _empty_kv(w, D, device)
        for b in range(w.B):
            for h in range(w.Hkv):
                d, s = kvgen.gen_kv_slab(w, which, b, h, threads)
                data[b, h].copy_(_t(d, "cpu"))
                if scale is not None:
                    if w.kv_dtype == "fp8":
                        scale[b, h] = float(s)
                    else:
                        scale[b, h].copy_(_t(s, "cpu"))
            if progress is not None:
                progress("generated %s for request %d/%d" % (which, b + 1, w.B))
        out[which] = (data, scale)
    return DeviceInputs(w, q, out["k"], out.get("v"), seq)
