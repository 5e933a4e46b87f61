"""GPU parity of the training pair: prism_fwd_ckpt (the forward pass that keeps
every chunk's start state) and prism_bwd_ckpt (the chunkwise backward reading
those checkpoints instead of recomputing them).

The forward's outputs equal prism_fwd_resume's; the checkpoints agree with the
chunk-start states the backward's own recompute writes to its workspace, on
every slot that holds a chunk; the gradients from the checkpoints match the
fp64 oracle's backward at the bf16 tolerance and agree with the recomputing
backward."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import BY_NAME
from gated_delta_rule_prologue_amd.inputs import f32_to_bf16_bits, make_inputs, to_float
from tests.gpu_common import TOL, max_rel, say, to_host
from tests.test_gpu_bwd import NAMES, W, check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()


def _up(x):
    return (x + 255) // 256 * 256


def _slots(inp):
    """Virtual-chunk slots that hold a chunk: floor(cu[n] / 64) + n + c."""
    cu = inp.cu_seqlens
    return [int(cu[n]) // 64 + n + c for n in range(inp.n_seqs)
            for c in range((int(cu[n + 1] - cu[n]) + 63) // 64)]


def _bf16_f64(raw_u8):
    return (raw_u8.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _go(inp, residual="linear", with_state=True, seed=4):
    """fwd_ckpt, then the backward from its checkpoints and recomputing; returns
    the forward outputs of both forwards, both gradient sets, the checkpoint
    bytes and the recompute's chunk-start states (from its workspace)."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    from tests.test_gpu_state import dev_tensor, start_state
    dev = binding.to_device(inp)
    rng = np.random.default_rng(seed)
    d_o_bits = f32_to_bf16_bits(rng.standard_normal((inp.total_tokens, inp.heads, inp.dv)).astype(np.float32))
    d_o = dev_tensor(d_o_bits)
    S0 = start_state(inp) if with_state else None
    dsf = rng.standard_normal((inp.n_seqs, inp.heads, inp.dk, inp.dv)).astype(np.float32) if with_state else None
    S0_t = dev_tensor(S0) if with_state else None
    dsf_t = dev_tensor(dsf) if with_state else None
    args = (dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"], dev["h"],
            dev["conv_w"], dev["cu_seqlens"], inp.L)
    o1, s1, ck = binding.fwd_ckpt(*args, S_init=S0_t, residual=residual)
    o2, s2, _ = binding.fwd_resume(*args, S_init=S0_t, residual=residual)
    gc = binding.bwd(*args, d_o, dS_final=dsf_t, S_init=S0_t, residual=residual, checkpoints=ck)
    d = binding.make_dims(inp.n_seqs, inp.total_tokens, inp.heads, inp.dk, inp.dv, binding.PRISM_BF16)
    ws = torch.zeros(int(binding.lib().prism_bwd_workspace_bytes(d, inp.L)), dtype=torch.uint8, device="cuda")
    gr = binding.bwd(*args, d_o, dS_final=dsf_t, S_init=S0_t, residual=residual, workspace=ws)
    torch.cuda.synchronize()
    host = lambda gs: {n: (to_host(gs[n]) if gs[n] is not None else None) for n in NAMES}
    # the recompute's chunk-start states in its workspace: after kw and the per-chunk matrices
    nv = (inp.total_tokens // 64 + inp.n_seqs) * inp.heads
    off = max(_up(inp.total_tokens * inp.heads * inp.dk * 2), 256) + _up(nv * 20480)
    half = _up(nv * inp.dk * inp.dv * 2)
    rec = ws[off:off + 2 * half].cpu().numpy()
    rec_kw = ws[:off].cpu().numpy()
    ref = oracle.bwd(inp, to_float(d_o_bits).astype(np.float64), dS_final=dsf, S_init=S0, residual=residual)
    return ((to_host(o1), to_host(s1)), (to_host(o2), to_host(s2)), host(gc), host(gr),
            ck.cpu().numpy(), rec, half, ref, rec_kw)


def _check_checkpoints(inp, ck, rec, half, rec_kw=None):
    """Both checkpoint arrays against the chunk-start states the recompute
    leaves in its workspace (rows, then transposes), on the slots that hold a
    chunk; the transposes against the rows; and the stored write keys bit for
    bit against the recompute's (the same prologue on the same inputs)."""
    H, dk, dv = inp.heads, inp.dk, inp.dv
    slots = _slots(inp)
    n = (inp.total_tokens // 64 + inp.n_seqs) * H * dk * dv
    rows = []
    for part in range(2):
        a = _bf16_f64(ck[part * half:(part + 1) * half])[:n].reshape(-1, H, dk * dv)
        b = _bf16_f64(rec[part * half:(part + 1) * half])[:n].reshape(-1, H, dk * dv)
        err = max_rel(a[slots], b[slots]) if slots else 0.0
        say(f"  checkpoints part {part}: {len(slots)} slots, max rel {err:.3e}")
        assert np.isfinite(a[slots]).all()
        assert err <= TOL["bf16"]
        rows.append(a[slots])
    if slots:
        t = rows[1].reshape(len(slots), H, dv, dk).transpose(0, 1, 3, 2).reshape(len(slots), H, dk * dv)
        assert np.array_equal(rows[0], t), "the two checkpoint arrays are not transposes"
    if rec_kw is not None:
        nkw = inp.total_tokens * H * dk * 2
        assert np.array_equal(ck[2 * half:2 * half + nkw], rec_kw[:nkw]), "checkpointed kw differs"


CASES = [
    W(dk=64, dv=64, L=4, lengths=(150, 1, 0, 70, 64)),
    W(dk=128, dv=128, L=4, lengths=(200, 65)),
    W(dk=64, dv=128, L=1, lengths=(90, 3)),
    W(dk=128, dv=64, L=8, lengths=(70, 129), H=3),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"dk{w.dk}-dv{w.dv}-L{w.L}")
def test_checkpointed_training_pair(w):
    inp = make_inputs(w)
    say(f"checkpointed pair {w}")
    (o1, s1), (o2, s2), gc, gr, ck, rec, half, ref, rec_kw = _go(inp)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2), "fwd_ckpt outputs differ from fwd_resume"
    _check_checkpoints(inp, ck, rec, half, rec_kw)
    check(gc, ref, "bf16")
    for n in NAMES:
        if gc[n] is not None and gr[n] is not None:
            assert max_rel(gc[n], gr[n]) <= TOL["bf16"], n


def test_checkpointed_pair_gelu_without_state():
    from tests.test_gpu_gelu import amplify
    inp = amplify(make_inputs(W(dk=128, dv=128, L=5, lengths=(200, 65))))
    (o1, s1), (o2, s2), gc, gr, ck, rec, half, ref, rec_kw = _go(inp, residual="gelu", with_state=False)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    _check_checkpoints(inp, ck, rec, half, rec_kw)
    check(gc, ref, "bf16")


def test_checkpointed_pair_lm_layer():
    """The LM layer at full size: checkpoints against the recompute's, every
    gradient against the recomputing backward (the oracle's full-size backward
    is covered on sampled chains elsewhere)."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    inp = make_inputs(BY_NAME["lm-130m-layer"])
    dev = binding.to_device(inp)
    rng = np.random.default_rng(8)
    from tests.test_gpu_state import dev_tensor
    d_o = dev_tensor(f32_to_bf16_bits(rng.standard_normal((inp.total_tokens, inp.heads, inp.dv)).astype(np.float32)))
    args = (dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"], dev["h"],
            dev["conv_w"], dev["cu_seqlens"], inp.L)
    o1, s1, ck = binding.fwd_ckpt(*args)
    o2, s2 = binding.fwd(*args)
    gc = binding.bwd(*args, d_o, checkpoints=ck, want_dS_init=False)
    d = binding.make_dims(inp.n_seqs, inp.total_tokens, inp.heads, inp.dk, inp.dv, binding.PRISM_BF16)
    ws = torch.zeros(int(binding.lib().prism_bwd_workspace_bytes(d, inp.L)), dtype=torch.uint8, device="cuda")
    gr = binding.bwd(*args, d_o, want_dS_init=False, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(o1), to_host(o2)) and np.array_equal(to_host(s1), to_host(s2))
    nv = (inp.total_tokens // 64 + inp.n_seqs) * inp.heads
    off = max(_up(inp.total_tokens * inp.heads * inp.dk * 2), 256) + _up(nv * 20480)
    half = _up(nv * inp.dk * inp.dv * 2)
    _check_checkpoints(inp, ck.cpu().numpy(), ws[off:off + 2 * half].cpu().numpy(), half,
                       ws[:off].cpu().numpy())
    for n in NAMES:
        if gc[n] is None or gr[n] is None:
            continue
        err = max_rel(to_host(gc[n]), to_host(gr[n]))
        say(f"  lm-130m-layer d{n}: checkpoints vs recompute {err:.3e}")
        assert err <= TOL["bf16"], (n, err)


# ----------------------------------------------------------------------------- bf16 gradients
BF16_GRADS = ("q", "k", "v", "u", "a", "h")


def _bf16_and_f32_grads(inp, residual="linear", with_state=True, seed=6):
    """The checkpoint backward on the same inputs and checkpoints, once with
    fp32 and once with bf16 token-sized gradients."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    from tests.test_gpu_state import dev_tensor, start_state
    dev = binding.to_device(inp)
    rng = np.random.default_rng(seed)
    d_o_bits = f32_to_bf16_bits(rng.standard_normal((inp.total_tokens, inp.heads, inp.dv)).astype(np.float32))
    d_o = dev_tensor(d_o_bits)
    S0 = start_state(inp) if with_state else None
    dsf = rng.standard_normal((inp.n_seqs, inp.heads, inp.dk, inp.dv)).astype(np.float32) if with_state else None
    S0_t = dev_tensor(S0) if with_state else None
    dsf_t = dev_tensor(dsf) if with_state else None
    args = (dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"], dev["h"],
            dev["conv_w"], dev["cu_seqlens"], inp.L)
    _, _, ck = binding.fwd_ckpt(*args, S_init=S0_t, residual=residual)
    kw = dict(dS_final=dsf_t, S_init=S0_t, residual=residual, checkpoints=ck)
    g32 = binding.bwd(*args, d_o, **kw)
    g16 = binding.bwd(*args, d_o, grad_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    return g32, g16, d_o_bits, S0, dsf


def _check_rounded(inp, g32, g16):
    """Each bf16 gradient is its fp32 twin rounded to nearest even, bit for bit
    (both come from the same fp32 arithmetic); the fp32-only gradients agree
    up to the arbitrary order of the LDS sums behind dg and db."""
    import torch
    for n in BF16_GRADS:
        if g32[n] is None:
            assert g16[n] is None
            continue
        assert g16[n].dtype == torch.bfloat16 and g16[n].shape == g32[n].shape
        got = g16[n].view(torch.int16).cpu().numpy().view(np.uint16)
        want = f32_to_bf16_bits(g32[n].cpu().numpy())
        bad = int(np.count_nonzero(got != want))
        say(f"  d{n}: {got.size} bf16 elements, {bad} differ from the rounded fp32 gradient")
        assert bad == 0, n
    for n in ("g", "b", "conv_w", "S_init"):
        if g32[n] is not None:
            assert g16[n].dtype == torch.float32
            assert max_rel(to_host(g16[n]), to_host(g32[n])) <= 1e-5, n


@pytest.mark.parametrize("w", CASES[:2] + CASES[3:], ids=lambda w: f"dk{w.dk}-dv{w.dv}-L{w.L}")
def test_bf16_gradients_are_the_rounded_fp32_ones(w):
    inp = make_inputs(w)
    say(f"bf16 gradients {w}")
    g32, g16, d_o_bits, S0, dsf = _bf16_and_f32_grads(inp)
    _check_rounded(inp, g32, g16)
    ref = oracle.bwd(inp, to_float(d_o_bits).astype(np.float64), dS_final=dsf, S_init=S0)
    check({n: (to_host(g16[n]) if g16[n] is not None else None) for n in NAMES}, ref, "bf16")


EDGE = [
    # the most levels, empty and one-token sequences, a chunk of 63 and of 65 tokens
    W(dk=64, dv=128, L=16, lengths=(1, 0, 200, 63, 65)),
    # whole chunks only, five heads, two levels
    W(dk=128, dv=64, L=2, lengths=(64, 64, 128), H=5),
    # forget gates near zero: the in-chunk decays underflow fp32
    W(dk=64, dv=64, L=6, lengths=(300, 17), g_mu=-3.0),
]


@pytest.mark.parametrize("w", EDGE, ids=["L16-ragged", "H5-whole-chunks", "strong-decay"])
def test_bf16_gradients_edge_shapes(w):
    inp = make_inputs(w)
    say(f"bf16 gradients, edge shape {w}")
    g32, g16, d_o_bits, S0, dsf = _bf16_and_f32_grads(inp)
    _check_rounded(inp, g32, g16)
    ref = oracle.bwd(inp, to_float(d_o_bits).astype(np.float64), dS_final=dsf, S_init=S0)
    check({n: (to_host(g16[n]) if g16[n] is not None else None) for n in NAMES}, ref, "bf16")


def test_bf16_gradients_gelu_one_level():
    """The GELU chain, and L = 1 (no u, a, h: only dq, dk, dv in bf16)."""
    from tests.test_gpu_gelu import amplify
    inp = amplify(make_inputs(W(dk=128, dv=128, L=5, lengths=(200, 65))))
    g32, g16, *_ = _bf16_and_f32_grads(inp, residual="gelu", with_state=False)
    _check_rounded(inp, g32, g16)
    inp = make_inputs(CASES[2])
    g32, g16, *_ = _bf16_and_f32_grads(inp)
    _check_rounded(inp, g32, g16)


def test_bf16_gradients_lm_layer():
    """The LM layer at full size (B=8, T=2048, H=6, d=128, L=4)."""
    inp = make_inputs(BY_NAME["lm-130m-layer"])
    g32, g16, *_ = _bf16_and_f32_grads(inp, with_state=False)
    _check_rounded(inp, g32, g16)


@pytest.mark.parametrize("name", ["recsys-history", "varlen-histories"])
def test_checkpointed_pair_full_size(name):
    """The recommendation histories (B=64, T=1024, H=4, d=64, L=4) and the
    variable-length batch (512 sequences, H=8, d=64, L=8) at full size: the
    checkpoint backward against the recomputing one on every gradient, and its
    bf16 gradients against its fp32 ones bit for bit."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    inp = make_inputs(BY_NAME[name])
    say(f"{name}: T={inp.total_tokens} chains={inp.n_seqs * inp.heads}")
    dev = binding.to_device(inp)
    rng = np.random.default_rng(8)
    from tests.test_gpu_state import dev_tensor
    d_o = dev_tensor(f32_to_bf16_bits(rng.standard_normal((inp.total_tokens, inp.heads, inp.dv)).astype(np.float32)))
    args = (dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"], dev["h"],
            dev["conv_w"], dev["cu_seqlens"], inp.L)
    o1, s1, ck = binding.fwd_ckpt(*args)
    o2, s2 = binding.fwd(*args)
    assert np.array_equal(to_host(o1), to_host(o2)) and np.array_equal(to_host(s1), to_host(s2))
    gc = binding.bwd(*args, d_o, checkpoints=ck, want_dS_init=False)
    gb = binding.bwd(*args, d_o, checkpoints=ck, want_dS_init=False, grad_dtype=torch.bfloat16)
    gr = binding.bwd(*args, d_o, want_dS_init=False)
    torch.cuda.synchronize()
    for n in NAMES:
        if gc[n] is None or gr[n] is None:
            continue
        err = max_rel(to_host(gc[n]), to_host(gr[n]))
        say(f"  {name} d{n}: checkpoints vs recompute {err:.3e}")
        assert err <= TOL["bf16"], (n, err)
    _check_rounded(inp, gc, gb)
