"""GPU parity of the fused write keys (PRISM_FUSED_KW=1): prism_fwd computes kw
inside the scan kernel instead of launching the prologue.

Checked against the fp64 oracle (every element of o and S_final), against the
two-kernel path, and for the path actually taken: the fused path never writes
the workspace's write-key region, so a sentinel there survives the call.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import BY_NAME, Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs
from tests.gpu_common import TOL, gpu_fwd, max_rel, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()


@pytest.fixture
def fused(monkeypatch):
    monkeypatch.setenv("PRISM_FUSED_KW", "1")


def W(H=2, dk=64, dv=64, L=4, lengths=(100,), seed=11, g_mu=3.0):
    return Workload("fk", heads=H, dk=dk, dv=dv, L=L, dtype="bf16", seed=seed,
                    lengths=list(lengths), g_mu=g_mu)


def _fwd_with_sentinel(inp):
    """prism_fwd with a workspace whose write-key region holds 0xA5 bytes;
    returns (o, S_final, whether that region is untouched)."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    dev = binding.to_device(inp)
    d = binding.make_dims(inp.n_seqs, inp.total_tokens, inp.heads, inp.dk, inp.dv, binding.PRISM_BF16)
    need = binding.workspace_bytes(d, inp.L)
    kwb = inp.total_tokens * inp.heads * inp.dk * 2
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    o, s = binding.fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"], dev["h"],
                       dev["conv_w"], dev["cu_seqlens"], inp.L, workspace=ws)
    torch.cuda.synchronize()
    untouched = bool((ws[:kwb] == 0xA5).all().item())
    return to_host(o), to_host(s), untouched


# dk = 64 at L = 4 and 8, dk = 128 at L = 4; sequences of 0 .. 4 chunks with
# ragged ends, sequence starts inside and at the edge of the conv window
CASES = [
    W(dk=64, L=4, lengths=(200, 64, 1, 0, 77, 2, 3)),
    W(dk=64, L=8, lengths=(129, 0, 5, 256)),
    W(dk=128, dv=128, L=4, lengths=(300, 63, 1, 65)),
    W(dk=128, dv=64, L=4, H=3, lengths=(190, 4)),
    W(dk=64, dv=128, L=4, lengths=(130,), g_mu=-2.0),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"dk{w.dk}-dv{w.dv}-L{w.L}-{len(w.lengths)}seq")
def test_fused_matches_oracle(w, fused):
    inp = make_inputs(w)
    o, s, untouched = _fwd_with_sentinel(inp)
    o_ref, s_ref = oracle.fwd(inp)
    eo, es = max_rel(o, o_ref), max_rel(s, s_ref)
    say(f"fused {w}: o {eo:.3e} S {es:.3e} kw region untouched {untouched}")
    assert untouched, "the fused path was not taken"
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("w", CASES[:3], ids=lambda w: f"dk{w.dk}-L{w.L}")
def test_fused_agrees_with_two_kernels(w, monkeypatch):
    """kw computed in the scan with the prologue's arithmetic: the outputs
    differ from the two-kernel path's by no more than rounding order."""
    inp = make_inputs(w)
    o2, s2 = gpu_fwd(inp)
    monkeypatch.setenv("PRISM_FUSED_KW", "1")
    o1, s1, untouched = _fwd_with_sentinel(inp)
    assert untouched
    say(f"fused vs two kernels: o {max_rel(o1, o2):.3e} S {max_rel(s1, s2):.3e}")
    assert max_rel(o1, o2) <= 1e-3 and max_rel(s1, s2) <= 1e-3


@pytest.mark.parametrize("w", [W(dk=64, L=3), W(dk=128, dv=128, L=8, H=1, lengths=(129,)),
                               W(dk=64, L=1)], ids=["L3", "dk128-L8", "L1"])
def test_unsupported_shapes_take_two_kernels(w, fused):
    """Shapes the fused kernel does not serve run the prologue as before."""
    inp = make_inputs(w)
    o, s, untouched = _fwd_with_sentinel(inp)
    o_ref, s_ref = oracle.fwd(inp)
    assert not untouched
    assert max_rel(o, o_ref) <= TOL["bf16"] and max_rel(s, s_ref) <= TOL["bf16"]


@pytest.mark.parametrize("name", ["recsys-history", "lm-130m-layer", "varlen-histories"])
def test_fused_workloads(name, fused):
    """The three workloads the fused path serves, at full size, every chain."""
    w = BY_NAME[name]
    inp = make_inputs(w)
    say(f"fused workload {name}: T={inp.total_tokens}")
    o, s, untouched = _fwd_with_sentinel(inp)
    o_ref, s_ref = oracle.fwd(inp)
    eo, es = max_rel(o, o_ref), max_rel(s, s_ref)
    say(f"fused workload {name}: o err {eo:.3e} S err {es:.3e}")
    assert untouched
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
