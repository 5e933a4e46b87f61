"""GPU parity of the carried-state entry points against the fp64 oracle:
prism_fwd_resume (start state S_init, conv history k_hist, history out) and
prism_decode_step (one token per sequence, state and history in place).

Small shapes compare every element; the serving-sized decode steps compare
every element as well (the oracle evaluates one token per chain).  The
carried history is compared bit for bit: it is a copy of k rows.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs, f32_to_bf16_bits
from tests.gpu_common import TOL, max_rel, say, to_host
from tests.test_gpu_parity import SCAN_KERNELS

pytestmark = pytest.mark.gpu
PER_TOKEN = ("q", "k", "v", "u", "a", "h", "g", "b")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()


def W(H=2, dk=64, dv=64, L=4, dtype="bf16", lengths=(100,), seed=21, g_mu=3.0):
    return Workload("state", heads=H, dk=dk, dv=dv, L=L, dtype=dtype, seed=seed,
                    lengths=list(lengths), g_mu=g_mu)


def start_state(inp, seed=3, scale=0.3):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((inp.n_seqs, inp.heads, inp.dk, inp.dv))).astype(np.float32)


def history(inp, seed=4):
    rng = np.random.default_rng(seed)
    x = (0.25 * rng.standard_normal((inp.n_seqs, inp.heads, 3, inp.dk))).astype(np.float32)
    return f32_to_bf16_bits(x) if inp.dtype == "bf16" else x


def dev_tensor(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def host_bits(t, dtype):
    """Raw storage of a device tensor, in the oracle's input form."""
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def gpu_resume(inp, S0, hist, in_place=False):
    import torch
    from gated_delta_rule_prologue_amd import binding
    dev = binding.to_device(inp)
    s0 = None if S0 is None else dev_tensor(S0)
    h0 = None if hist is None else dev_tensor(hist)
    hout = h0 if (in_place and h0 is not None) else torch.full(
        (inp.n_seqs, inp.heads, 3, inp.dk), float("nan"), device="cuda",
        dtype=torch.bfloat16 if inp.dtype == "bf16" else torch.float32)
    o, s, hout = binding.fwd_resume(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"],
                                    dev["a"], dev["h"], dev["conv_w"], dev["cu_seqlens"], inp.L,
                                    S_init=s0, k_hist=h0, S_final=s0 if in_place else None,
                                    k_hist_out=hout)
    torch.cuda.synchronize()
    return to_host(o), to_host(s), host_bits(hout, inp.dtype)


def check_resume(inp, S0, hist, in_place=False):
    o, s, hout = gpu_resume(inp, S0, hist, in_place)
    o_ref, s_ref = oracle.fwd(inp, S_init=S0, k_hist=hist)
    eo, es = max_rel(o, o_ref), max_rel(s, s_ref)
    say(f"  o err {eo:.3e}  S err {es:.3e}")
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL[inp.dtype] and es <= TOL[inp.dtype]
    want = oracle.k_history(inp, hist)
    got = hout.astype(np.float64) if inp.dtype == "f32" else to_host_bits(hout)
    assert np.array_equal(got, want)


def to_host_bits(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


RESUME_CASES = [
    W(dtype="f32", dk=64, dv=64, L=2, lengths=(130, 1, 2, 0, 64)),
    W(dtype="f32", dk=128, dv=128, L=4, lengths=(90, 1, 0, 65)),       # token-recurrent fp32
    W(dtype="bf16", dk=64, dv=64, L=4, lengths=(200, 1, 2, 3, 0, 65)),
    W(dtype="bf16", dk=128, dv=128, L=4, lengths=(150, 2, 64)),
    W(dtype="bf16", dk=128, dv=64, L=1, lengths=(70, 1)),
    W(dtype="bf16", dk=64, dv=128, L=8, lengths=(129, 0, 3)),
]


@pytest.mark.parametrize("w", RESUME_CASES,
                         ids=lambda w: f"{w.dtype}-dk{w.dk}-dv{w.dv}-L{w.L}-{len(w.lengths)}seq")
def test_fwd_resume_matches_oracle(w):
    inp = make_inputs(w)
    say(f"fwd_resume {w}")
    check_resume(inp, start_state(inp), history(inp))


@pytest.mark.parametrize("kernel", list(SCAN_KERNELS))
@pytest.mark.parametrize("dk", [64, 128])
def test_fwd_resume_every_scan_kernel(dk, kernel, monkeypatch):
    """The start state enters every bf16 scan kernel (slices of 16 and 32
    columns for the wavefront-specialised kernels, 32 for the two-pass scan,
    32 and 64 for the others)."""
    for key, val in SCAN_KERNELS[kernel].items():
        monkeypatch.setenv(key, val)
    slices = ([16, 32] if kernel.startswith("specialised") else [32] if kernel == "twopass"
              else [32, 64])
    inp = make_inputs(W(dtype="bf16", dk=dk, dv=64, L=3, lengths=(140, 3, 0, 64, 65)))
    for dvs in slices:
        monkeypatch.setenv("PRISM_DV_SLICE", str(dvs))
        say(f"fwd_resume kernel={kernel} dk={dk} dvs={dvs}")
        check_resume(inp, start_state(inp), history(inp))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_resume_in_place(dtype):
    """S_final written over S_init and the history over itself."""
    inp = make_inputs(W(dtype=dtype, lengths=(90, 1, 0, 2, 64)))
    say(f"fwd_resume in place {dtype}")
    check_resume(inp, start_state(inp), history(inp), in_place=True)


def test_fwd_resume_without_carry_equals_fwd():
    """No start state and no history: the same results as prism_fwd."""
    from tests.gpu_common import gpu_fwd
    inp = make_inputs(W(dtype="bf16", lengths=(100, 5)))
    o1, s1 = gpu_fwd(inp)
    o2, s2, _ = gpu_resume(inp, None, None)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def pieces(inp, cut):
    cu = inp.cu_seqlens
    lo_rows, hi_rows, c1, c2 = [], [], [0], [0]
    for n in range(inp.n_seqs):
        a, b = int(cu[n]), int(cu[n + 1])
        m = min(cut, b - a)
        lo_rows += range(a, a + m)
        hi_rows += range(a + m, b)
        c1.append(c1[-1] + m)
        c2.append(c2[-1] + b - a - m)

    def take(rows, c):
        idx = np.asarray(rows, dtype=np.int64)
        return dataclasses.replace(inp, cu_seqlens=np.asarray(c, dtype=np.int32),
                                   **{f: np.ascontiguousarray(getattr(inp, f)[idx])
                                      for f in PER_TOKEN if getattr(inp, f) is not None})

    return take(lo_rows, c1), take(hi_rows, c2), np.asarray(lo_rows), np.asarray(hi_rows)


@pytest.mark.parametrize("cut", [2, 64, 100])
def test_two_pieces_equal_one_call(cut):
    """Each sequence run in two calls, carrying S_final and k_hist_out from the
    first into the second, matches the oracle over the whole sequence."""
    inp = make_inputs(W(dtype="bf16", dk=128, dv=128, lengths=(250, 70, 1)))
    first, second, r1, r2 = pieces(inp, cut)
    o1, s1, h1 = gpu_resume(first, None, None)
    o2, s2, _ = gpu_resume(second, s1.astype(np.float32), h1)
    o_ref, s_ref = oracle.fwd(inp)
    o = np.zeros_like(o_ref)
    o[r1], o[r2] = o1, o2
    eo, es = max_rel(o, o_ref), max_rel(s2, s_ref)
    say(f"cut {cut}: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


# ----------------------------------------------------------------------------- decode
def step_inputs(inp, rows):
    """One token per sequence: the given rows of a multi-token input."""
    return dataclasses.replace(
        inp, cu_seqlens=np.arange(len(rows) + 1, dtype=np.int32),
        **{f: np.ascontiguousarray(getattr(inp, f)[rows]) for f in PER_TOKEN
           if getattr(inp, f) is not None})


def gpu_decode(step, S_dev, h_dev):
    import torch
    from gated_delta_rule_prologue_amd import binding
    dev = binding.to_device(step)
    o = binding.decode_step(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"],
                            dev["h"], dev["conv_w"], step.L, S_dev, h_dev)
    torch.cuda.synchronize()
    return to_host(o)


DECODE_CASES = [
    W(dtype="f32", dk=64, dv=64, L=2, lengths=(1,) * 5),
    W(dtype="bf16", dk=64, dv=64, L=4, lengths=(1,) * 7),
    W(dtype="bf16", dk=128, dv=128, L=4, lengths=(1,) * 3),
    W(dtype="bf16", dk=64, dv=128, L=1, lengths=(1,) * 2),
    W(dtype="f32", dk=128, dv=64, L=16, lengths=(1,) * 4),
]


@pytest.mark.parametrize("w", DECODE_CASES,
                         ids=lambda w: f"{w.dtype}-dk{w.dk}-dv{w.dv}-L{w.L}-{len(w.lengths)}seq")
def test_decode_step_matches_oracle(w):
    step = make_inputs(w)
    S0, hist = start_state(step), history(step)
    say(f"decode {w}")
    S_dev, h_dev = dev_tensor(S0), dev_tensor(hist)
    o = gpu_decode(step, S_dev, h_dev)
    o_ref, s_ref, h_ref = oracle.decode_step(step, S0, hist)
    eo, es = max_rel(o, o_ref), max_rel(to_host(S_dev), s_ref)
    say(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]
    got = host_bits(h_dev, w.dtype)
    got = got.astype(np.float64) if w.dtype == "f32" else to_host_bits(got)
    assert np.array_equal(got, h_ref)


def test_prefill_then_decode_equals_one_call():
    """fwd_resume over the first 70 tokens, then 12 decode steps, carrying the
    state and history on the device: the oracle over all 82 tokens."""
    import torch
    inp = make_inputs(W(dtype="bf16", dk=128, dv=128, L=4, lengths=(82, 82, 82)))
    first, _, r1, _ = pieces(inp, 70)
    from gated_delta_rule_prologue_amd import binding
    dev = binding.to_device(first)
    hist = torch.zeros((3, 2, 3, 128), dtype=torch.bfloat16, device="cuda")
    _, S, _ = binding.fwd_resume(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"],
                                 dev["a"], dev["h"], dev["conv_w"], dev["cu_seqlens"], inp.L,
                                 k_hist_out=hist)
    o_ref, s_ref = oracle.fwd(inp)
    worst = 0.0
    for t in range(70, 82):
        rows = inp.cu_seqlens[:-1] + t
        o = gpu_decode(step_inputs(inp, rows), S, hist)
        worst = max(worst, max_rel(o, o_ref[rows]))
    es = max_rel(to_host(S), s_ref)
    say(f"prefill + decode: o err {worst:.3e}  S err {es:.3e}")
    assert worst <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("shape", [(512, 8, 64, 64, 8), (8, 6, 128, 128, 4), (64, 4, 64, 64, 4)],
                         ids=["recsys-512x8-d64-L8", "lm-8x6-d128-L4", "recsys-64x4-d64-L4"])
def test_decode_serving_shapes(shape):
    """Serving-sized decode steps, every element, from a state with the scale
    of a long history (the S_final of a 256-token prefill is of the same order)."""
    n, H, dk, dv, L = shape
    step = make_inputs(W(H=H, dk=dk, dv=dv, L=L, lengths=(1,) * n, seed=31))
    S0, hist = start_state(step, scale=1.0), history(step)
    say(f"decode serving shape {shape}")
    S_dev, h_dev = dev_tensor(S0), dev_tensor(hist)
    o = gpu_decode(step, S_dev, h_dev)
    o_ref, s_ref, h_ref = oracle.decode_step(step, S0, hist)
    eo, es = max_rel(o, o_ref), max_rel(to_host(S_dev), s_ref)
    say(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert np.array_equal(to_host_bits(host_bits(h_dev, "bf16")), h_ref)
