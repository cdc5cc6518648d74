"""GPU: the autograd wrapper (FrozenExpertMLP) is the explicit forward and
input-gradient calls, bit for bit, and leaves the frozen weights without a
gradient."""
import numpy as np
import pytest
import torch

import workload

pytestmark = pytest.mark.gpu


def test_autograd_wrapper_matches_explicit_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    c = workload.custom_case([40, 0, 300, 7], 128, 96, seed=61)
    dev = torch.device("cuda:0")
    off = torch.from_numpy(np.ascontiguousarray(c.offsets)).to(dev)
    packed = gg.gg_pack_weights(c.w1.to(dev), c.w2.to(dev))
    dy = c.dy.to(dev)
    x = c.x.to(dev).requires_grad_(True)
    y = gg.FrozenExpertMLP.apply(x, off, packed, c.E, c.H, c.F)
    y.backward(dy)
    h1, a = gg.gg_forward_fc1_swiglu(c.x.to(dev), off, packed, c.E, c.H, c.F)
    y_ref = gg.gg_forward_fc2(a, off, packed, c.E, c.H, c.F)
    dx_ref = gg.gg_dgrad(dy, h1, off, packed, c.E, c.H, c.F)
    torch.cuda.synchronize()
    assert torch.equal(y.detach().view(torch.int16), y_ref.view(torch.int16))
    assert torch.equal(x.grad.view(torch.int16), dx_ref.view(torch.int16))
    assert not packed.requires_grad and packed.grad is None
