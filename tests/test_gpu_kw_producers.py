"""GPU parity of the in-scan write-key producers (PRISM_KW_PRODUCERS=1, bf16
at the shapes they serve): producer workgroups in the scan launch form kw chunk
by chunk and flag each chunk, and the scan reads a chunk's keys once flagged.

Checked against the fp64 oracle (every element of o and S_final), against the
two-launch path (prologue, then scan: PRISM_KW_PRODUCERS=0; the same arithmetic,
so equal up to the compiler's rounding order of the write keys), and for
the path actually taken: each of a producer block's eight wavefronts counts
its part of a (virtual chunk, head) into that item's flag in the workspace, so
the flags end at 8 for every item that holds tokens and 0 for the others,
while the two-launch path leaves that region as it was.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import BY_NAME, Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs
from tests.gpu_common import TOL, max_rel, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()


def W(H=2, dk=64, dv=64, L=4, lengths=(100,), seed=13, g_mu=3.0):
    return Workload("kp", heads=H, dk=dk, dv=dv, L=L, dtype="bf16", seed=seed,
                    lengths=list(lengths), g_mu=g_mu)


def _expected_flags(inp):
    """8 (the producer wavefronts) at slot (floor(cu[n] / 64) + n + c) * H + e
    for every chunk c of every non-empty sequence n and head e; 0 elsewhere."""
    H, cu = inp.heads, inp.cu_seqlens
    f = np.zeros((inp.total_tokens // 64 + inp.n_seqs) * H, dtype=np.int32)
    for n in range(inp.n_seqs):
        for c in range((int(cu[n + 1] - cu[n]) + 63) // 64):
            base = (int(cu[n]) // 64 + n + c) * H
            f[base:base + H] = 8
    return f


def _fwd(inp, producers, dev=None):
    """prism_fwd with a workspace pre-filled with 0xA5; returns o, S_final,
    the write keys and the flag region as the call left them."""
    import os
    import torch
    from gated_delta_rule_prologue_amd import binding
    os.environ["PRISM_KW_PRODUCERS"] = "1" if producers else "0"
    try:
        dev = dev or binding.to_device(inp)
        d = binding.make_dims(inp.n_seqs, inp.total_tokens, inp.heads, inp.dk, inp.dv, binding.PRISM_BF16)
        need = binding.workspace_bytes(d, inp.L)
        kwb = (inp.total_tokens * inp.heads * inp.dk * 2 + 255) // 256 * 256
        nfl = (inp.total_tokens // 64 + inp.n_seqs) * inp.heads
        if producers:
            assert need == kwb + (4 * nfl + 255) // 256 * 256
        ws = torch.full((max(need, kwb + 4 * nfl),), 0xA5, dtype=torch.uint8, device="cuda")
        o, s = binding.fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"],
                           dev["h"], dev["conv_w"], dev["cu_seqlens"], inp.L, workspace=ws)
        torch.cuda.synchronize()
        kw = ws[:inp.total_tokens * inp.heads * inp.dk * 2].cpu().numpy().copy()
        flags = ws[kwb:kwb + 4 * nfl].cpu().numpy().view(np.int32).copy()
        return to_host(o), to_host(s), kw, flags
    finally:
        del os.environ["PRISM_KW_PRODUCERS"]


# dk = 64 at L = 4 and 8, dk = 128 at L = 4, dv 64 and 128; sequences of 0 .. 4
# chunks with ragged ends, sequence starts inside and at the edge of the conv
# window, strong decay
CASES = [
    W(dk=64, L=4, lengths=(200, 64, 1, 0, 77, 2, 3)),
    W(dk=64, L=8, lengths=(129, 0, 5, 256)),
    W(dk=128, dv=128, L=4, lengths=(300, 63, 1, 65)),
    W(dk=128, dv=64, L=4, H=3, lengths=(190, 4)),
    W(dk=64, dv=128, L=4, lengths=(130,), g_mu=-2.0),
    W(dk=128, dv=128, L=4, H=4, lengths=(1000, 1, 640, 333)),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"dk{w.dk}-dv{w.dv}-L{w.L}-{len(w.lengths)}seq")
def test_producers_match_oracle(w):
    inp = make_inputs(w)
    o, s, _, flags = _fwd(inp, True)
    o_ref, s_ref = oracle.fwd(inp)
    eo, es = max_rel(o, o_ref), max_rel(s, s_ref)
    say(f"kw producers {w}: o {eo:.3e} S {es:.3e}")
    assert np.array_equal(flags, _expected_flags(inp)), "the producer path was not taken as designed"
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def _kw_f32(raw):
    return (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _agree(kw1, kw2, o1, o2, s1, s2, what):
    """Write keys within one bf16 unit in the last place of each other (the two
    kernels evaluate the same formula, contracted into FMAs by the compiler in
    its own order); outputs within the bf16 tolerance (a key one unit apart
    moves the outputs of the tokens after it)."""
    a, b = _kw_f32(kw1), _kw_f32(kw2)
    ulp = np.abs(a - b) / np.maximum(np.maximum(np.abs(a), np.abs(b)), 1e-30)
    say(f"  {what}: kw equal {np.array_equal(kw1, kw2)}, max rel {ulp.max():.2e}; "
        f"o {max_rel(o1, o2):.2e} S {max_rel(s1, s2):.2e}")
    assert ulp.max() <= 2.0 ** -7, "write keys differ by more than one bf16 ulp"
    assert max_rel(o1, o2) <= TOL["bf16"] and max_rel(s1, s2) <= TOL["bf16"]


@pytest.mark.parametrize("w", CASES[:4], ids=lambda w: f"dk{w.dk}-dv{w.dv}-L{w.L}")
def test_producers_agree_with_two_launches(w):
    """The producers use the prologue's arithmetic and the scan is the same
    kernel: write keys, outputs and final states agree with the
    prologue-then-scan path's up to rounding order."""
    inp = make_inputs(w)
    o1, s1, kw1, f1 = _fwd(inp, True)
    o2, s2, kw2, f2 = _fwd(inp, False)
    assert np.array_equal(f1, _expected_flags(inp))
    assert (f2.view(np.uint32) == 0xA5A5A5A5).all(), "the two-launch path touched the flags"
    _agree(kw1, kw2, o1, o2, s1, s2, f"{w}")


def test_producers_lm_layer():
    """The LM layer (B=8, T=2048, H=6, d=128, L=4): 192 scan workgroups and 64
    producers; every chain against the oracle, and against the two launches."""
    inp = make_inputs(BY_NAME["lm-130m-layer"])
    o, s, kw, flags = _fwd(inp, True)
    assert np.array_equal(flags, _expected_flags(inp))
    o2, s2, kw2, _ = _fwd(inp, False)
    _agree(kw, kw2, o, o2, s, s2, "lm-130m-layer")
    o_ref, s_ref = oracle.fwd(inp)
    eo, es = max_rel(o, o_ref), max_rel(s, s_ref)
    say(f"kw producers lm-130m-layer: o {eo:.3e} S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("name,w", [("lm-130m-layer", None), ("ragged", CASES[5]), ("dk64-L8", CASES[1])])
def test_scan_saw_the_produced_keys(name, w):
    """No chunk's keys were read before they were stored: the scan run alone
    (prism_scan) on the keys the producers left in the workspace gives
    bit-identical outputs and final states."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    inp = make_inputs(BY_NAME[name] if w is None else w)
    dev = binding.to_device(inp)
    o1, s1, kw, _ = _fwd(inp, True, dev)
    kwt = torch.from_numpy(kw.view(np.int16).reshape(inp.total_tokens, inp.heads, inp.dk).copy())
    kwt = kwt.view(torch.bfloat16).to("cuda")
    o2, s2 = binding.scan(dev["q"], dev["k"], kwt, dev["v"], dev["g"], dev["b"], dev["cu_seqlens"])
    torch.cuda.synchronize()
    o2, s2 = to_host(o2), to_host(s2)
    say(f"  {name}: o equal {np.array_equal(o1, o2)} ({max_rel(o1, o2):.2e}), "
        f"S equal {np.array_equal(s1, s2)} ({max_rel(s1, s2):.2e})")
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_repeated_calls_reuse_the_workspace(monkeypatch):
    """Three calls in a row on one workspace (the flags are cleared by each
    call): the same results every time."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    monkeypatch.setenv("PRISM_KW_PRODUCERS", "1")
    inp = make_inputs(W(dk=128, dv=128, L=4, H=2, lengths=(500, 70)))
    dev = binding.to_device(inp)
    d = binding.make_dims(inp.n_seqs, inp.total_tokens, inp.heads, inp.dk, inp.dv, binding.PRISM_BF16)
    ws = torch.zeros(binding.workspace_bytes(d, inp.L), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        o, s = binding.fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"],
                           dev["h"], dev["conv_w"], dev["cu_seqlens"], inp.L, workspace=ws)
        torch.cuda.synchronize()
        outs.append((to_host(o), to_host(s)))
    for o, s in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(s, outs[0][1])
