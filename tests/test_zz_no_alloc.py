"""prism_fwd_noalloc (the forward pass with the library's static scratch as
workspace, for callers that cannot allocate) against prism_fwd: the same
kernels, so the same bits, on two calls in a row -- the LM layer at full size
(B=8, T=2048, H=6, d=128, L=4), then a smaller ragged batch that reuses the
scratch the first call left behind."""
import numpy as np
import pytest

from gated_delta_rule_prologue_amd.configs import BY_NAME, Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs
from tests.gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()


def _both(inp):
    import torch
    from gated_delta_rule_prologue_amd import binding
    dev = binding.to_device(inp)
    args = (dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"], dev["h"],
            dev["conv_w"], dev["cu_seqlens"], inp.L)
    o_ref, s_ref = binding.fwd(*args)
    o = torch.full_like(o_ref, float("nan"))
    s = torch.full_like(s_ref, float("nan"))
    binding.fwd_noalloc(*args, o=o, S_final=s)
    torch.cuda.synchronize()
    return o, s, o_ref, s_ref


def test_fwd_noalloc_equals_fwd_twice():
    big = make_inputs(BY_NAME["lm-130m-layer"])
    small = make_inputs(Workload("small", heads=3, dk=64, dv=128, L=3, dtype="bf16", seed=8,
                                 lengths=[200, 0, 1, 65]))
    for name, inp in (("lm-130m-layer", big), ("small ragged", small)):
        say(f"fwd_noalloc {name}")
        o, s, o_ref, s_ref = _both(inp)
        assert o.shape == o_ref.shape and s.shape == s_ref.shape
        assert np.array_equal(o.float().cpu().numpy(), o_ref.float().cpu().numpy()), name
        assert np.array_equal(s.cpu().numpy(), s_ref.cpu().numpy()), name


def test_fwd_noalloc_rejects_oversize_shape():
    """One 65,536-token sequence of 16 heads needs more than the static scratch:
    PRISM_ENOSPACE, before anything is launched."""
    import ctypes
    from gated_delta_rule_prologue_amd import binding as B
    d = B.make_dims(1, 65536, 16, 128, 128, B.PRISM_BF16)
    assert B.workspace_bytes(d, 4) > B.NOALLOC_MAX_BYTES
    fake = 0x10000
    rc = B.lib().prism_fwd_noalloc(ctypes.byref(d), *([fake] * 10), 4, fake, fake, None)
    assert rc == B.PRISM_ENOSPACE
