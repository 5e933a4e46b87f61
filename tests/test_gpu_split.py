"""GPU parity of the split scan for few, long sequences: each sequence cut into
P segments scanned side by side (local scans and transition-only scans in one
launch), chained through the segment transitions and corrected, against the
fp64 oracle.  The split is forced with PRISM_SPLIT at sizes the oracle
evaluates in full; the long-context workload takes it on its own (full-size
parity of that workload is in test_gpu_parity.py)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import BY_NAME, Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs
from tests.gpu_common import TOL, gpu_fwd, max_rel, say, to_host
from tests.test_gpu_state import dev_tensor, history, host_bits, start_state, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()


def W(H=2, dk=64, dv=64, L=4, lengths=(700, 300, 65, 1, 0, 129), seed=51, g_mu=3.0):
    return Workload("split", heads=H, dk=dk, dv=dv, L=L, dtype="bf16", seed=seed,
                    lengths=list(lengths), g_mu=g_mu)


@pytest.mark.parametrize("P", [2, 3, 5])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_split_matches_oracle(dk, dv, P, monkeypatch):
    """Segments of whole chunks, ragged last segments, empty ones (sequences
    shorter than P chunks, an empty sequence), all compared in full."""
    monkeypatch.setenv("PRISM_SPLIT", str(P))
    inp = make_inputs(W(dk=dk, dv=dv))
    say(f"split P={P} dk={dk} dv={dv}")
    o, s = gpu_fwd(inp)
    o_ref, s_ref = oracle.fwd(inp)
    eo, es = max_rel(o, o_ref), max_rel(s, s_ref)
    say(f"  o err {eo:.3e}  S err {es:.3e}")
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_split_strong_decay_long(monkeypatch):
    """A long chain with fast forgetting: the carried state must decay through
    the segment transitions exactly as through the chunks."""
    monkeypatch.setenv("PRISM_SPLIT", "4")
    inp = make_inputs(W(dk=128, dv=128, H=1, lengths=(3000, 1500), g_mu=0.0))
    o, s = gpu_fwd(inp)
    o_ref, s_ref = oracle.fwd(inp)
    eo, es = max_rel(o, o_ref), max_rel(s, s_ref)
    say(f"split strong decay: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("in_place", [False, True])
def test_split_with_carried_state(in_place, monkeypatch):
    """A start state enters the first segment through the correction as well."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    monkeypatch.setenv("PRISM_SPLIT", "3")
    inp = make_inputs(W(dk=128, dv=128, lengths=(900, 64, 0, 130)))
    S0, hist = start_state(inp), history(inp)
    dev = binding.to_device(inp)
    s0 = dev_tensor(S0)
    h0 = dev_tensor(hist)
    hout = h0 if in_place else torch.empty_like(h0)
    o, s, hout = binding.fwd_resume(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"],
                                    dev["a"], dev["h"], dev["conv_w"], dev["cu_seqlens"], inp.L,
                                    S_init=s0, k_hist=h0, S_final=s0 if in_place else None,
                                    k_hist_out=hout)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd(inp, S_init=S0, k_hist=hist)
    eo, es = max_rel(to_host(o), o_ref), max_rel(to_host(s), s_ref)
    say(f"split resume in_place={in_place}: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert np.array_equal(to_host_bits(host_bits(hout, "bf16")), oracle.k_history(inp, hist))


def test_split_deterministic(monkeypatch):
    monkeypatch.setenv("PRISM_SPLIT", "2")
    inp = make_inputs(W(dk=128, dv=128))
    o1, s1 = gpu_fwd(inp)
    o2, s2 = gpu_fwd(inp)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_long_context_takes_the_split():
    """The 64k workload (16 chains) splits on its own: its workspace holds the
    segment buffers on top of the write keys."""
    from gated_delta_rule_prologue_amd import binding
    w = BY_NAME["long-context-64k"]
    d = binding.make_dims(1, 65536, w.heads, w.dk, w.dv, binding.PRISM_BF16)
    kw = 65536 * w.heads * w.dk * 2
    assert binding.workspace_bytes(d, w.L) > kw
    lm = BY_NAME["lm-130m-layer"]
    d2 = binding.make_dims(8, 16384, lm.heads, lm.dk, lm.dv, binding.PRISM_BF16)
    # the LM layer does not split: the write keys only (the fused scan needs no scratch)
    assert binding.scan_workspace_bytes(d2) == 0
    assert binding.workspace_bytes(d2, lm.L) == 16384 * lm.heads * lm.dk * 2
