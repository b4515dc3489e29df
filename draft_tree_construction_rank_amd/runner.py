"""Round runner: moves a synthetic instance to the GPU and calls the C ABI.

Argument marshalling only: every computation happens in libdtree.so.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import binding as B


def _dt(dtype: str) -> int:
    return B.DT_BF16 if dtype == "bf16" else B.DT_F32


def _torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def params_for(inst, *, R: Optional[int] = None, k: Optional[int] = None,
               Ncap: Optional[int] = None, mode: Optional[str] = None,
               temperature: Optional[float] = None, round_: Optional[int] = None,
               cond: Optional[int] = None) -> B.dt_params:
    m = inst.mode if mode is None else mode
    return B.make_params(R=inst.R if R is None else R, B=inst.B, k=inst.k if k is None else k,
                         V=inst.V, r=inst.r, Ncap=inst.Ncap if Ncap is None else Ncap,
                         logits_dtype=_dt(inst.dtype), head_dtype=_dt(inst.dtype),
                         mode=B.DT_SAMPLE if m == "sample" else B.DT_GREEDY,
                         temperature=inst.temperature if temperature is None else temperature,
                         cal=inst.cal, seed=inst.seed,
                         round_=inst.round if round_ is None else round_,
                         cond=getattr(inst, "cond", 0) if cond is None else cond)


@dataclasses.dataclass
class DeviceInputs:
    L: torch.Tensor
    U: torch.Tensor
    Wt: torch.Tensor
    root_token: torch.Tensor
    n_budget: torch.Tensor
    tau: torch.Tensor


def to_device(inst, device="cuda", *, n_budget=None, tau=None) -> DeviceInputs:
    td = _torch_dtype(inst.dtype)
    L = torch.from_numpy(np.ascontiguousarray(inst.L)).to(device=device, dtype=td).contiguous()
    U = torch.from_numpy(inst.U).to(device=device, dtype=td).contiguous()
    Wt = torch.from_numpy(inst.Wt).to(device=device, dtype=td).contiguous()
    nb = inst.n_budget if n_budget is None else np.broadcast_to(np.int32(n_budget), inst.R)
    ta = inst.tau if tau is None else np.broadcast_to(np.float32(tau), inst.R)
    return DeviceInputs(L=L, U=U, Wt=Wt,
                        root_token=torch.from_numpy(inst.root_token.astype(np.int32)).to(device),
                        n_budget=torch.from_numpy(np.ascontiguousarray(nb, np.int32)).to(device),
                        tau=torch.from_numpy(np.ascontiguousarray(ta, np.float32)).to(device))


def target_to_device(inst, target: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(target)).to(device=device,
                                                             dtype=_torch_dtype(inst.dtype))


def tree_to_numpy(t: dict) -> dict:
    out = {k: v.cpu().numpy() for k, v in t.items()}
    out["mask"] = out.pop("anc_mask").view(np.uint64)
    return out


class Round:
    """Holds parameters, workspace and outputs for repeated calls on one stream."""

    def __init__(self, inst, device="cuda", **pkw):
        self.p = params_for(inst, **pkw)
        self.ws = B.alloc_workspace(self.p, device)
        self.tree = B.alloc_tree(self.p, device)
        self.vout = B.alloc_verify(self.p, device)

    def build(self, d: DeviceInputs, stream=None) -> dict:
        B.tree_build(self.p, d.L, d.U, d.Wt, d.root_token, d.n_budget, d.tau, self.tree,
                     self.ws, stream)
        return self.tree

    def verify_greedy(self, target: torch.Tensor, stream=None) -> dict:
        B.tree_verify_greedy(self.p, self.tree, target, self.vout, self.ws, stream)
        return self.vout

    def verify_sample(self, d: DeviceInputs, target: torch.Tensor, stream=None) -> dict:
        B.tree_verify_sample(self.p, self.tree, d.L, d.U, d.Wt, d.root_token, target, self.vout,
                             self.ws, stream)
        return self.vout
