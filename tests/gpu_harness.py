"""Runs a drawn case through the HIP path (tests and benchmark helpers).

Only marshalling: upload the case, pack the weights with gg_pack_weights,
call the three entry points on the current stream.
"""
from __future__ import annotations

import sys

import numpy as np
import torch


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceCase:
    def __init__(self, case, device="cuda:0"):
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
        torch.cuda.synchronize()
        del w1, w2

    def forward(self, save_h1=True, h1_out=None, a_out=None, y=None):
        gg = self.gg
        h1, a = gg.gg_forward_fc1_swiglu(self.x, self.offsets, self.packed, self.E, self.H, self.F,
                                         save_h1=save_h1, h1_out=h1_out, a_out=a_out)
        y = gg.gg_forward_fc2(a, self.offsets, self.packed, self.E, self.H, self.F, y=y)
        return h1, a, y

    def dgrad(self, h1, workspace=None, dx=None):
        gg = self.gg
        if workspace is None:
            workspace = torch.empty(self.M, 2 * self.F, dtype=torch.bfloat16, device=self.dev)
        dx = gg.gg_dgrad(self.dy, h1, self.offsets, self.packed, self.E, self.H, self.F,
                         workspace=workspace, dx=dx)
        return workspace, dx
