"""Runs a drawn case through the HIP path (tests and benchmark helpers).

Only marshalling: upload the case, pack the weights with gg_pack_weights
(and, with frag=True, the opt-in fragment-ordered copies with gg_pack_frag),
call the entry points on the current stream.
"""
from __future__ import annotations

import sys

import numpy as np
import torch


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceCase:
    def __init__(self, case, device="cuda:0", frag: bool = False):
        import moe_expert_grouped_ragged_amd as gg
        self.gg = gg
        self.case = case
        self.E, self.H, self.F, self.M = case.E, case.H, case.F, case.M
        self.dev = torch.device(device)
        self.x = case.x.to(self.dev)
        self.dy = case.dy.to(self.dev)
        self.offsets = torch.from_numpy(np.ascontiguousarray(case.offsets)).to(self.dev)
        w1 = case.w1.to(self.dev)
        w2 = case.w2.to(self.dev)
        self.packed = gg.gg_pack_weights(w1, w2)
        self.frag = gg.gg_pack_frag(self.packed, self.E, self.H, self.F) if frag else None
        torch.cuda.synchronize()
        del w1, w2

    def forward(self, save_h1=True, h1_out=None, a_out=None, y=None):
        gg = self.gg
        if self.frag is None:
            h1, a = gg.gg_forward_fc1_swiglu(self.x, self.offsets, self.packed, self.E, self.H, self.F,
                                             save_h1=save_h1, h1_out=h1_out, a_out=a_out)
        else:
            h1, a = gg.gg_forward_fc1_glu(self.x, self.offsets, self.packed, self.E, self.H, self.F,
                                          save_h1=save_h1, h1_out=h1_out, a_out=a_out, frag=self.frag)
        y = gg.gg_forward_fc2_frag(a, self.offsets, self.packed, self.frag, self.E, self.H, self.F, y=y)
        return h1, a, y

    def dgrad(self, h1, workspace=None, dx=None):
        gg = self.gg
        if workspace is None:
            workspace = torch.empty(self.M, 2 * self.F, dtype=torch.bfloat16, device=self.dev)
        if self.frag is None:
            dx = gg.gg_dgrad(self.dy, h1, self.offsets, self.packed, self.E, self.H, self.F,
                             workspace=workspace, dx=dx)
        else:
            dx, _ = gg.gg_dgrad_glu(self.dy, h1, self.offsets, self.packed, self.E, self.H, self.F,
                                    want_dprobs=False, workspace=workspace, dx=dx, frag=self.frag)
        return workspace, dx


def layouts(H: int, F: int):
    """The weight layouts a shape can run: the packed buffer alone, and with
    the opt-in fragment-ordered copies when the shape has them."""
    import moe_expert_grouped_ragged_amd as gg
    return (False, True) if gg.has_frag(H, F) else (False,)


def bitwise_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))
