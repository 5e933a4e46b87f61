"""The autograd wrapper (gated_delta_rule_prologue_amd.autograd.prism): loss.backward()
gives the gradients of the fp64 oracle's backward for every input and the
start state, in each input's dtype, on each of its routes: prism_fwd_ckpt then
prism_bwd_ckpt with bf16 gradients (the default), prism_fwd_ckpt then the
recomputing backward when the token walk is forced (PRISM_BWD_CHUNKED=0, which
prism_bwd_ckpt refuses), and prism_fwd_resume then prism_bwd_ex when the
environment selects a scan kernel prism_fwd_ckpt does not run
(PRISM_SCAN_SPECIALISED=0)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import Workload
from gated_delta_rule_prologue_amd.inputs import f32_to_bf16_bits, make_inputs, to_float
from tests.gpu_common import TOL, max_rel, say
from tests.test_gpu_state import dev_tensor, start_state

pytestmark = pytest.mark.gpu
FIELDS = ("q", "k", "v", "u", "g", "b", "a", "h", "conv_w")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()


ROUTES = {"checkpoints": {}, "token-walk": {"PRISM_BWD_CHUNKED": "0"},
          "recompute": {"PRISM_SCAN_SPECIALISED": "0"}}


@pytest.mark.parametrize("residual,use_state,route", [("linear", True, "checkpoints"),
                                                      ("gelu", True, "checkpoints"),
                                                      ("linear", False, "checkpoints"),
                                                      ("linear", True, "token-walk"),
                                                      ("gelu", True, "recompute")])
def test_autograd_matches_oracle(residual, use_state, route, monkeypatch):
    import torch
    for name, value in ROUTES[route].items():
        monkeypatch.setenv(name, value)
    from gated_delta_rule_prologue_amd import binding
    from gated_delta_rule_prologue_amd.autograd import prism
    w = Workload("ag", heads=2, dk=64, dv=64, L=3, dtype="bf16", seed=81, lengths=[90, 1, 0, 40])
    inp = make_inputs(w)
    if residual == "gelu":
        from tests.test_gpu_gelu import amplify
        inp = amplify(inp)
    dev = binding.to_device(inp)
    leaves = {n: dev[n].clone().requires_grad_(True) for n in FIELDS}
    S0 = start_state(inp)
    S0_t = dev_tensor(S0).requires_grad_(True)
    rng = np.random.default_rng(6)
    d_o = to_float(f32_to_bf16_bits(rng.standard_normal(dev["v"].shape).astype(np.float32)))
    dsf = rng.standard_normal((inp.n_seqs, inp.heads, inp.dk, inp.dv)).astype(np.float32)
    o, S = prism(*(leaves[n] for n in FIELDS), dev["cu_seqlens"], inp.L,
                 S_init=S0_t, residual=residual)
    loss = (o.float() * torch.from_numpy(d_o).cuda()).sum()
    if use_state:
        loss = loss + (S * torch.from_numpy(dsf).cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    ref = oracle.bwd(inp, d_o.astype(np.float64), dS_final=dsf if use_state else None, S_init=S0,
                     residual=residual)
    for n in FIELDS + ("S_init",):
        src = S0_t if n == "S_init" else leaves[n]
        got = src.grad
        assert got is not None, n
        assert got.dtype == src.dtype and got.shape == src.shape, n
        err = max_rel(got.float().cpu().numpy(), ref[n])
        say(f"{route} {residual} state={use_state} d{n} err {err:.3e}")
        assert err <= TOL["bf16"], (n, err)
