"""The C-ABI entry points under HIP graph capture: every launch they make is a
kernel on the caller's stream (no allocation, no memset, no host
synchronisation), so a graph captured around them replays them.  Each test
replays several times with eager work and synchronisations in between, and
checks every replay against the same calls made eagerly."""
import numpy as np
import pytest

from gated_delta_rule_prologue_amd.configs import Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs
from tests.gpu_common import say, to_host
from tests.test_gpu_state import dev_tensor, history, start_state

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()


def W(H=2, dk=64, dv=64, L=4, lengths=(1,) * 16, seed=61):
    return Workload("graph", heads=H, dk=dk, dv=dv, L=L, dtype="bf16", seed=seed, lengths=list(lengths))


def test_decode_steps_replay_from_a_graph():
    """Four decode steps (different tokens, state and history carried in place)
    captured once and replayed three times from saved starting states."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    steps = [binding.to_device(make_inputs(W(seed=61 + i))) for i in range(4)]
    L = 4
    S0 = dev_tensor(start_state(make_inputs(W())))
    h0 = dev_tensor(history(make_inputs(W())))
    S, h = S0.clone(), h0.clone()
    outs = [torch.empty_like(st["v"]) for st in steps]

    def run():
        for st, o in zip(steps, outs):
            binding.decode_step(st["q"], st["k"], st["v"], st["u"], st["g"], st["b"], st["a"],
                                st["h"], st["conv_w"], L, S, h, o=o)

    # eager reference from the same start
    run()
    torch.cuda.synchronize()
    ref_o = [to_host(o) for o in outs]
    ref_S, ref_h = to_host(S), h.clone()
    # capture (warm-up on a side stream first, as graph capture requires)
    S.copy_(S0); h.copy_(h0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        S.copy_(S0); h.copy_(h0)
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref_o):
            assert np.array_equal(to_host(o), r), rep
        assert np.array_equal(to_host(S), ref_S) and torch.equal(h, ref_h), rep
        say(f"replay {rep}: identical to eager")


@pytest.mark.parametrize("split", ["0", "2"])
def test_forward_replays_from_a_graph(split, monkeypatch):
    """prism_fwd (prologue and scan; with PRISM_SPLIT=2 the split scan's plan,
    paired scan, combine and correction) captured and replayed."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    monkeypatch.setenv("PRISM_SPLIT", split)
    inp = make_inputs(W(dk=128, dv=128, lengths=(700, 130, 1)))
    dev = binding.to_device(inp)
    d = binding.Dims(inp.n_seqs, inp.total_tokens, inp.heads, inp.dk, inp.dv, binding.PRISM_BF16)
    ws = torch.empty(binding.workspace_bytes(d, inp.L), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(dev["v"])
    S = torch.empty((inp.n_seqs, inp.heads, inp.dk, inp.dv), dtype=torch.float32, device="cuda")

    def run():
        binding.fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"], dev["h"],
                    dev["conv_w"], dev["cu_seqlens"], inp.L, o=o, S_final=S, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref_o, ref_S = to_host(o), to_host(S)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        o.zero_(); S.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(o), ref_o) and np.array_equal(to_host(S), ref_S), rep
    say(f"split={split}: three replays identical to eager")


def test_backward_replays_from_a_graph():
    """prism_bwd_ex (write-key recomputation, zero fills, scan backward,
    write-key backward) captured once and replayed three times into outputs
    poisoned with NaN before each replay.  dv and dS_init are written once per
    element and must equal the eager call bit for bit; the gradients summed
    with fp32 atomics over value slices (dq, dk, dg, db, dconv_w, and through
    dkw du, da, dh) only up to the order of those sums."""
    import ctypes
    import torch
    from gated_delta_rule_prologue_amd import binding
    inp = make_inputs(W(dk=64, dv=64, L=3, lengths=(150, 1, 0, 70)))
    dev = binding.to_device(inp)
    T, H, dk, dv, L, n = inp.total_tokens, inp.heads, inp.dk, inp.dv, inp.L, inp.n_seqs
    gen = torch.Generator(device="cuda").manual_seed(3)
    dO = torch.randn(dev["v"].shape, device="cuda", generator=gen).to(torch.bfloat16)
    dsf = torch.randn((n, H, dk, dv), device="cuda", generator=gen)
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {"q": torch.empty((T, H, dk), **f32), "k": torch.empty((T, H, dk), **f32),
           "v": torch.empty((T, H, dv), **f32), "u": torch.empty((T, H, L - 1, dk), **f32),
           "g": torch.empty((T, H), **f32), "b": torch.empty((T, H), **f32),
           "a": torch.empty((T, H, L - 1, dk), **f32), "h": torch.empty((T, H, L - 1, dk), **f32),
           "conv_w": torch.empty((H, dk, 4), **f32), "S_init": torch.empty((n, H, dk, dv), **f32)}
    d = binding.Dims(n, T, H, dk, dv, binding.PRISM_BF16)
    lib = binding.lib()
    need = int(lib.prism_bwd_workspace_bytes(ctypes.byref(d), L))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def call(stream):
        return lib.prism_bwd_ex(
            ctypes.byref(d), P(dev["q"]), P(dev["k"]), P(dev["v"]), P(dev["u"]), P(dev["g"]),
            P(dev["b"]), P(dev["a"]), P(dev["h"]), P(dev["conv_w"]), P(dev["cu_seqlens"]), L, 0,
            None, P(dO), P(dsf), P(out["q"]), P(out["k"]), P(out["v"]), P(out["u"]), P(out["g"]),
            P(out["b"]), P(out["a"]), P(out["h"]), P(out["conv_w"]), P(out["S_init"]), P(ws),
            need, ctypes.c_void_p(stream))

    assert call(torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    ref = {k: v.cpu().numpy() for k, v in out.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert call(side.cuda_stream) == 0
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert call(torch.cuda.current_stream().cuda_stream) == 0
    for rep in range(3):
        for t in out.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in out.items():
            got = t.cpu().numpy()
            assert np.isfinite(got).all(), (rep, name)
            if name in ("v", "S_init"):
                assert np.array_equal(got, ref[name]), (rep, name)
            else:
                scale = max(float(np.max(np.abs(ref[name]))), 1e-30)
                assert float(np.max(np.abs(got - ref[name]))) <= 1e-5 * scale, (rep, name)
        say(f"backward replay {rep}: dv, dS_init identical to eager, the rest within 1e-5")


def test_training_pair_replays_from_a_graph():
    """prism_fwd_ckpt then prism_bwd_ckpt with bf16 gradients, captured in one
    graph (the binding's output tensors come from the graph's pool) and
    replayed three times into outputs poisoned with NaN before each replay.
    o, S_final, dS_init and the six bf16 gradients are computed without
    atomics and must equal the eager calls bit for bit; dg, db and dconv_w
    only up to the order of their sums."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    inp = make_inputs(W(dk=128, dv=128, L=3, lengths=(150, 1, 0, 70)))
    dev = binding.to_device(inp)
    n, H, dk, dv = inp.n_seqs, inp.heads, inp.dk, inp.dv
    gen = torch.Generator(device="cuda").manual_seed(5)
    dO = torch.randn(dev["v"].shape, device="cuda", generator=gen).to(torch.bfloat16)
    S0 = dev_tensor(start_state(inp))
    dsf = torch.randn((n, H, dk, dv), device="cuda", generator=gen)
    args = (dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"], dev["h"],
            dev["conv_w"], dev["cu_seqlens"], inp.L)

    def pair():
        o, S, ck = binding.fwd_ckpt(*args, S_init=S0)
        g = binding.bwd(*args, dO, dS_final=dsf, S_init=S0, checkpoints=ck, grad_dtype=torch.bfloat16)
        return {"o": o, "S_final": S, **{n_: t for n_, t in g.items() if t is not None}}

    def host(t):
        return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()

    ref = {k: host(t) for k, t in pair().items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pair()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = pair()
    assert set(out) == set(ref)
    for rep in range(3):
        for t in out.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in out.items():
            got = host(t)
            if name in ("g", "b", "conv_w"):
                assert np.isfinite(got).all(), (rep, name)
                scale = max(float(np.max(np.abs(ref[name]))), 1e-30)
                assert float(np.max(np.abs(got - ref[name]))) <= 1e-5 * scale, (rep, name)
            else:
                assert np.array_equal(got, ref[name]), (rep, name)
        say(f"training pair replay {rep}: o, S_final, dS_init and the bf16 gradients identical to eager")
